// bf16 KV-cached decode on the gfx950 matrix cores: split-history attention
// followed by a merge of the partial softmax states.
//
// One query per sequence attends to its cache (B, h_kv, T_cap, d_h) in place;
// query head a reads cache head g(a) = floor(a / r) through the index, the
// cache is never duplicated per query head ([EffSeq] 缓存字节; [MhaMqaGqa]
// section 8: reading the same K/V once per query head would bring the traffic
// back to the multi-head level).  A workgroup owns one (sequence, K/V head,
// chunk of up to 32 query heads of the group, slice of the history): every
// K/V byte of the slice is read from HBM once and serves all r query heads of
// the group as the 32 columns of one matrix-core tile ([MhaMqaGqa] section 7:
// the 4-row decode group shares one K/V tile).  Decode has few rows, so the
// history is split across workgroups to fill the chip ([MhaMqaGqa] section 9),
// and each slice yields a partial state (m, l, u) that the combine kernel
// merges with the rule of [AttnVar] 3.5:
//     m' = max_s m_s,   l = sum_s e^{m_s - m'} l_s,   u = sum_s e^{m_s - m'} u_s,   o = u / l.
// Inside a workgroup the 4 waves take interleaved 32-key blocks of each
// 128-key tile and merge their states in LDS at the end.
#include "internal.h"
#include "mfma_common.h"

namespace gqa {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 128;          // keys per workgroup tile (32 per wave)
constexpr int kTargetWG = 512;      // workgroups the split heuristic aims for (2 resident per CU)
constexpr int kMinChunk = 256;      // smallest history slice per workgroup

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* seq_lens;
  const int32_t* q_pos;
  void* o;
  float* ws_u;        // [B][h_q][n_split_cap][D] unnormalized partial outputs
  float* ws_ml;       // [B][h_q][n_split_cap][2]  (m * c, l) per partial
  int h_q, h_kv, r, hc_count, T_cap, max_len;
  int chunk, n_split, n_split_cap;
  int direct;         // one split: write the normalized output directly
  float c;            // scale * log2(e)
};

template <int D>
struct DecodeLds {
  static constexpr int KS = D * 2 + 16;
  static constexpr int VS = D * 2 + 32;
  static constexpr int K_BYTES = kTile * KS;
  static constexpr int STAGE = K_BYTES + kTile * VS;
  // the end-of-slice merge reuses the stage: 4 waves x 32 rows x D floats + (m, l)
  static constexpr int MERGE = 4 * 32 * D * 4 + 4 * 32 * 2 * 4;
  static constexpr int TOTAL = STAGE > MERGE ? STAGE : MERGE;
};

__device__ __forceinline__ int visible_end(const DecodeParams& p, int b) {
  const int len = clampi(p.seq_lens[b], 0, p.T_cap);
  const int pos = p.q_pos ? p.q_pos[b] : len - 1;
  int e = min(len, pos + 1);
  e = min(e, p.max_len);
  return max(e, 0);
}

template <int D, bool OUT_BF16>
__global__ void __launch_bounds__(kThreads, 2)
decode_bf16_kernel(DecodeParams p) {
  using L = DecodeLds<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int col = lane & 31;

  const int split = blockIdx.x;
  const int g = blockIdx.y / p.hc_count;
  const int hcix = blockIdx.y % p.hc_count;
  const int b = blockIdx.z;

  const int kv_end = visible_end(p, b);
  const int lo = split * p.chunk;
  const int hi = min(lo + p.chunk, kv_end);
  const int n_heads_here = min(32, p.r - hcix * 32);

  if (lo >= hi) {
    // empty slice: only the single-split path owes an output (zeros)
    if (p.direct) {
      for (int e = tid; e < n_heads_here * D; e += kThreads) {
        const int j = e / D, d = e % D;
        const int head = g * p.r + hcix * 32 + j;
        const size_t oi = (size_t)(b * p.h_q + head) * D + d;
        if constexpr (OUT_BF16) static_cast<uint16_t*>(p.o)[oi] = 0;
        else static_cast<float*>(p.o)[oi] = 0.f;
      }
    }
    return;
  }

  // query column = one query head of the group (zero beyond the group's heads)
  const bool col_valid = col < n_heads_here;
  const int head_col = g * p.r + hcix * 32 + col;
  bf16x8 qf[D / 16];
  {
    const uint16_t* qrow = p.q + (size_t)(b * p.h_q + head_col) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (col_valid) x = *reinterpret_cast<const uint4*>(qrow + ks * 16 + h * 8);
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const size_t kv_base = (size_t)(b * p.h_kv + g) * p.T_cap * D;
  const uint32_t slice_bytes = (uint32_t)hi * D * 2;          // keys >= hi read as zeros
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + kv_base, slice_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + kv_base, slice_bytes);

  constexpr int UNITS = kTile * D / 8 / kThreads;           // 16-byte chunks per thread per tensor
  uint4 kreg[UNITS], vreg[UNITS];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < UNITS; ++i) {
      const int u = tid + kThreads * i;
      const int row = u / (D / 8), c8 = u % (D / 8);
      const uint32_t off = (uint32_t)((k0 + row) * D + c8 * 8) * 2;
      kreg[i] = load16(krs, off);
      vreg[i] = load16(vrs, off);
    }
  };
  auto store_tile = [&]() {
    unsigned char* vs_ = lds + L::K_BYTES;
#pragma unroll
    for (int i = 0; i < UNITS; ++i) {
      const int u = tid + kThreads * i;
      const int row = u / (D / 8), c8 = u % (D / 8);
      *reinterpret_cast<uint4*>(lds + row * L::KS + c8 * 16) = kreg[i];
      *reinterpret_cast<uint4*>(vs_ + row * L::VS + c8 * 16) = vreg[i];
    }
  };

  const int n_tiles = (hi - lo + kTile - 1) / kTile;
  load_tile(lo);
  for (int t = 0; t < n_tiles; ++t) {
    const int k0 = lo + t * kTile;
    lds_barrier();                 // every wave is done reading the previous tile
    store_tile();
    if (t + 1 < n_tiles) load_tile(k0 + kTile);
    lds_barrier();                 // tile t is in LDS

    const unsigned char* vs_ = lds + L::K_BYTES;
    const int kw = wave * 32;      // this wave's 32-key block of the tile
    f32x16 sacc;
#pragma unroll
    for (int kd = 0; kd < D / 16; ++kd) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds + (kw + col) * L::KS + (kd * 16 + h * 8) * 2);
      sacc = mfma32(a, qf[kd], kd == 0 ? f32x16{} : sacc);
    }
    if (k0 + kTile > hi) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + kw + 8 * (e >> 2) + 4 * h + (e & 3);
        sacc[e] = key < hi ? sacc[e] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[e]);
    mx = pair_max(mx);
    const bool grow = (mx - m_run) * p.c > kLazyRescale;     // false for -inf - (-inf)
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? fast_exp2((m_run - mx) * p.c) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
      m_run = grow ? mx : m_run;
    }
    const float mc = (m_run == -INFINITY ? 0.f : m_run) * p.c;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pe = fast_exp2(fmaf(sacc[e], p.c, -mc));
      sacc[e] = pe;
      psum += pe;
    }
    l_run += psum;
    bf16x8 pf[2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int e0 = 8 * c2;
      pf[c2] = pack_bf16x8(sacc[e0], sacc[e0 + 1], sacc[e0 + 2], sacc[e0 + 3],
                           sacc[e0 + 4], sacc[e0 + 5], sacc[e0 + 6], sacc[e0 + 7]);
    }
    // chunks of this wave's block: kc = 2 * wave + c2 of the tile
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const bf16x8 a = load_vt_operand(vs_, L::VS, 2 * wave + c2, db * 32, lane);
        oacc[db] = mfma32(a, pf[c2], oacc[db]);
      }
  }

  // ---- merge the 4 waves' states in LDS
  lds_barrier();
  float* mo = reinterpret_cast<float*>(lds);              // [wave][D][32]
  float* mml = mo + 4 * D * 32;                            // [wave][32][2]
  const float l_pair = pair_sum(l_run);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int d = db * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
      mo[(wave * D + d) * 32 + col] = oacc[db][e];
    }
  if (h == 0) {
    mml[(wave * 32 + col) * 2 + 0] = (m_run == -INFINITY) ? -INFINITY : m_run * p.c;
    mml[(wave * 32 + col) * 2 + 1] = l_pair;
  }
  lds_barrier();

  // thread -> (row j, d range): 32 rows x D values, D / 8 per thread
  const int j = tid & 31;
  const int dgrp = tid >> 5;             // 0..7
  float mw[4], M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) { mw[w] = mml[(w * 32 + j) * 2]; M = fmaxf(M, mw[w]); }
  float wgt[4], lsum = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wgt[w] = (mw[w] == -INFINITY) ? 0.f : fast_exp2(mw[w] - M);
    lsum += wgt[w] * mml[(w * 32 + j) * 2 + 1];
  }
  if (j < n_heads_here) {
    const int head = g * p.r + hcix * 32 + j;
    if (p.direct) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        const int d = dgrp * (D / 8) + i;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) acc += wgt[w] * mo[(w * D + d) * 32 + j];
        const size_t oi = (size_t)(b * p.h_q + head) * D + d;
        if constexpr (OUT_BF16) {
          __bf16 x = (__bf16)(acc * inv);
          static_cast<uint16_t*>(p.o)[oi] = __builtin_bit_cast(uint16_t, x);
        } else {
          static_cast<float*>(p.o)[oi] = acc * inv;
        }
      }
    } else {
      const size_t pidx = (size_t)(b * p.h_q + head) * p.n_split_cap + split;
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        const int d = dgrp * (D / 8) + i;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) acc += wgt[w] * mo[(w * D + d) * 32 + j];
        p.ws_u[pidx * D + d] = acc;
      }
      if (dgrp == 0) {
        p.ws_ml[pidx * 2 + 0] = M;
        p.ws_ml[pidx * 2 + 1] = lsum;
      }
    }
  }
}

// Merge the partial states of one (sequence, query head): [AttnVar] 3.5 applied
// split after split.  One wave per output row.
template <int D, bool OUT_BF16>
__global__ void __launch_bounds__(64)
decode_combine_kernel(DecodeParams p) {
  const int head = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int kv_end = visible_end(p, b);
  const int n = (kv_end + p.chunk - 1) / p.chunk;
  const size_t base = (size_t)(b * p.h_q + head) * p.n_split_cap;
  constexpr int PER = D / 64;
  float M = -INFINITY, Lsum = 0.f, U[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) U[i] = 0.f;
  for (int s = 0; s < n; ++s) {
    const float ms = p.ws_ml[(base + s) * 2];
    const float ls = p.ws_ml[(base + s) * 2 + 1];
    if (ms == -INFINITY) continue;
    const float Mn = fmaxf(M, ms);
    const float a = fast_exp2(M - Mn);       // 0 on the first live split
    const float w = fast_exp2(ms - Mn);
    Lsum = a * Lsum + w * ls;
#pragma unroll
    for (int i = 0; i < PER; ++i) U[i] = a * U[i] + w * p.ws_u[(base + s) * D + lane + 64 * i];
    M = Mn;
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const size_t oi = (size_t)(b * p.h_q + head) * D + lane + 64 * i;
    if constexpr (OUT_BF16) {
      __bf16 x = (__bf16)(U[i] * inv);
      static_cast<uint16_t*>(p.o)[oi] = __builtin_bit_cast(uint16_t, x);
    } else {
      static_cast<float*>(p.o)[oi] = U[i] * inv;
    }
  }
}

template <int D, bool OUT_BF16>
hipError_t launch_t(const DecodeParams& prm, int B, hipStream_t s) {
  constexpr int smem = DecodeLds<D>::TOTAL;
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_bf16_kernel<D, OUT_BF16>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  dim3 grid(prm.n_split, prm.h_kv * prm.hc_count, B);
  hipLaunchKernelGGL((decode_bf16_kernel<D, OUT_BF16>), grid, dim3(kThreads), smem, s, prm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || prm.direct) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D, OUT_BF16>), dim3(prm.h_q, B), dim3(64), 0, s, prm);
  return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode_bf16(int B, int h_q, int h_kv, int T_cap, int D, int len) {
  DecodePlan pl;
  const int r = h_q / h_kv;
  pl.head_chunks = (r + 31) / 32;
  const long long pairs = (long long)B * h_kv * pl.head_chunks;
  long long cap = (kTargetWG + pairs - 1) / pairs;
  if (cap < 1) cap = 1;
  const long long max_cap = (T_cap + kMinChunk - 1) / kMinChunk;
  if (cap > max_cap) cap = max_cap < 1 ? 1 : max_cap;
  pl.n_split_cap = (int)cap;
  if (len < 1) len = 1;
  long long chunk = (len + cap - 1) / cap;
  chunk = (chunk + kTile - 1) / kTile * kTile;
  if (chunk < kMinChunk) chunk = kMinChunk;
  pl.chunk = (int)chunk;
  pl.n_split = (int)((len + chunk - 1) / chunk);
  pl.workspace_bytes = (pl.n_split > 1 || cap > 1)
      ? (size_t)B * h_q * cap * ((size_t)D + 2) * sizeof(float) : 0;
  return pl;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, const DecodePlan& pl, hipStream_t s) {
  DecodeParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.seq_lens = a.seq_lens;
  p.q_pos = a.q_pos;
  p.o = a.o;
  p.h_q = a.h_q; p.h_kv = a.h_kv; p.r = a.h_q / a.h_kv;
  p.hc_count = pl.head_chunks;
  p.T_cap = a.T_cap; p.max_len = a.max_len;
  p.chunk = pl.chunk; p.n_split = pl.n_split; p.n_split_cap = pl.n_split_cap;
  p.direct = pl.n_split == 1 ? 1 : 0;
  p.c = a.scale * kLog2e;
  const size_t u_bytes = (size_t)a.B * a.h_q * pl.n_split_cap * a.D * sizeof(float);
  p.ws_u = static_cast<float*>(a.workspace);
  p.ws_ml = a.workspace ? reinterpret_cast<float*>(static_cast<char*>(a.workspace) + u_bytes) : nullptr;
  if (a.D == 128) return a.out_bf16 ? launch_t<128, true>(p, a.B, s) : launch_t<128, false>(p, a.B, s);
  return a.out_bf16 ? launch_t<64, true>(p, a.B, s) : launch_t<64, false>(p, a.B, s);
}

}  // namespace gqa
