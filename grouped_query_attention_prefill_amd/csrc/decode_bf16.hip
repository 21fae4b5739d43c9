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
// Inside a workgroup the 4 waves take interleaved key blocks of each tile and
// merge their states in LDS at the end.  Groups of up to 16 query heads use
// 16x16 matrix-core tiles (16 keys per wave per 64-key tile), which halves the
// accumulator registers so that more workgroups share a CU and keep more HBM
// requests in flight; larger groups use 32x32 tiles over 128-key tiles.
// Grid rows take the sequences longest first.  The 16x16 kernel can also do the
// decode step's append ([AttnVar] 3.1: the new token's K/V are written, then all
// visible rows are read): the workgroup whose tiles hold the new row writes it
// and reads the new values in its place.  The ROPE instances rotate Q (and the
// appended key) as they load them.
#include "internal.h"
#include "mfma_common.h"
#include "rope_common.h"

namespace gqa {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 128;          // keys per workgroup tile (32 per wave)
constexpr int kTargetWG = 512;      // workgroups the split heuristic aims for (2 resident per CU;
                                    // the 16x16 kernel aims for four times as many: two rounds of
                                    // 4 resident per CU, so short sequences fill in behind long ones)
constexpr int kMinChunk = 256;      // smallest history slice per workgroup
constexpr int kPreferChunk = 4096;  // slice length the 16x16 kernel streams well
constexpr int kManySplits = 8;      // above this many splits the batched merge kernel runs

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
  int interleave;     // splits take interleaved tiles instead of contiguous slices
  // paged cache: pages (n_pages, h_kv, page_size, D); token j of sequence b is row
  // j % page_size of page block_table[b * max_pages + j / page_size]; null = contiguous
  const int32_t* block_table;
  int page_size, max_pages, n_pages;
  // fused append (16x16 kernel; write_pos null = none): row write_pos[b] of cache
  // head (b, g) receives k_new / v_new (B, h_kv, 1, D) before the decode reads it
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* write_pos;
  float c;            // scale * log2(e)
  int rope;           // the ROPE kernels: Q (and the appended key) rotated as loaded
  RopeTheta rope_theta;
};

// Position of sequence b's query (rotary encoding of Q): q_pos[b], else its last row.
__device__ __forceinline__ int query_position(const DecodeParams& p, int b) {
  return p.q_pos ? p.q_pos[b] : clampi(p.seq_lens[b], 0, p.T_cap) - 1;
}

// Elements 8 c8 .. 8 c8 + 7 of the key row appended to (b, g), rotated at position
// wp in the ROPE kernels (each 16-byte chunk also reads its partner chunk, d/2 away).
template <int D, bool ROPE>
__device__ __forceinline__ uint4 new_key_chunk(const DecodeParams& p, int b, int g, int c8, int wp) {
  const uint16_t* src = p.k_new + (size_t)(b * p.h_kv + g) * D;
  uint4 x = *reinterpret_cast<const uint4*>(src + c8 * 8);
  if constexpr (ROPE) {
    constexpr int HC = D / 16;                 // 16-byte chunks per half row
    const bool lo = c8 < HC;
    const uint4 y = *reinterpret_cast<const uint4*>(src + (lo ? c8 + HC : c8 - HC) * 8);
    bf16x8 a = __builtin_bit_cast(bf16x8, lo ? x : y), u = __builtin_bit_cast(bf16x8, lo ? y : x);
    const int i0 = (lo ? c8 : c8 - HC) * 8;
    uint64_t th[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) th[e] = p.rope_theta.t[i0 + e];
    rope_rotate8(a, u, wp, th);
    x = __builtin_bit_cast(uint4, lo ? a : u);
  }
  return x;
}

// The end of a workgroup: its 4 waves' states of HN query heads, held in LDS as
// mo [wave][head][D + 4] (unnormalized outputs; rows padded so that the float4
// reads below meet distinct banks) and mml [wave][head][2] (m * c, l), are merged
// with the rule of [AttnVar] 3.5 and stored: the normalized output when the slice
// is the whole history, else the partial state (m, l, u) for the combine kernel.
// Each half-wave takes one head and covers its D values in float4 units, so every
// store writes whole rows of contiguous memory.
template <int D>
constexpr int merge_stride() { return D + 4; }
template <int D, int HN>
constexpr int merge_bytes() { return 4 * HN * merge_stride<D>() * 4 + 4 * HN * 2 * 4; }

template <int D, int HN, bool OUT_BF16>
__device__ __forceinline__ void merge_and_store(const DecodeParams& p, const float* mo, const float* mml, int b,
                                                int head0, int n_heads, int split, int tid) {
  constexpr int MS = merge_stride<D>();
  static_assert(D / 4 <= 32, "one half-wave covers a head's row");
  const int dq = tid & 31;                  // float4 unit of the row (D / 4 of them)
  if (dq >= D / 4) return;
#pragma unroll
  for (int rnd = 0; rnd < HN / 8; ++rnd) {
    const int j = rnd * 8 + (tid >> 5);     // head of the workgroup
    if (j >= n_heads) continue;
    float mw[4], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) { mw[w] = mml[(w * HN + j) * 2]; M = fmaxf(M, mw[w]); }
    float wgt[4], lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wgt[w] = (mw[w] == -INFINITY) ? 0.f : fast_exp2(mw[w] - M);
      lsum += wgt[w] * mml[(w * HN + j) * 2 + 1];
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4 u = *reinterpret_cast<const float4*>(mo + (w * HN + j) * MS + 4 * dq);
      acc.x += wgt[w] * u.x; acc.y += wgt[w] * u.y; acc.z += wgt[w] * u.z; acc.w += wgt[w] * u.w;
    }
    const int head = head0 + j;
    if (p.direct) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      const size_t oi = (size_t)(b * p.h_q + head) * D + 4 * dq;
      if constexpr (OUT_BF16) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 w4;
        w4[0] = (__bf16)(acc.x * inv); w4[1] = (__bf16)(acc.y * inv);
        w4[2] = (__bf16)(acc.z * inv); w4[3] = (__bf16)(acc.w * inv);
        *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(p.o) + oi) = w4;
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(p.o) + oi) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
      }
    } else {
      const size_t pidx = (size_t)(b * p.h_q + head) * p.n_split_cap + split;
      *reinterpret_cast<float4*>(p.ws_u + pidx * D + 4 * dq) = acc;
      if (dq == 0) *reinterpret_cast<float2*>(p.ws_ml + pidx * 2) = make_float2(M, lsum);
    }
  }
}

template <int D>
struct DecodeLds {
  static constexpr int KS = D * 2 + 16;
  static constexpr int VS = D * 2 + 32;
  static constexpr int K_BYTES = kTile * KS;
  static constexpr int STAGE = K_BYTES + kTile * VS;
  // the end-of-slice merge reuses the stage: 4 waves x 32 rows x D floats + (m, l)
  static constexpr int MERGE = merge_bytes<D, 32>();
  static constexpr int TOTAL = STAGE > MERGE ? STAGE : MERGE;
};

__device__ __forceinline__ int visible_end(const DecodeParams& p, int b) {
  const int len = clampi(p.seq_lens[b], 0, p.T_cap);
  const int pos = p.q_pos ? p.q_pos[b] : len - 1;
  int e = min(len, pos + 1);
  e = min(e, p.max_len);
  return max(e, 0);
}

// The sequence that grid row z serves: sequences ranked by visible length, longest
// first (ties by index).  The dispatcher starts workgroups in grid order, so the
// longest histories are spread over the chip first and short ones fill in behind
// them instead of leaving a few long ones to stream alone at the end.  Batches
// larger than the workgroup keep their natural order.
__device__ __forceinline__ int sequence_of_rank(const DecodeParams& p, int z, int B, int tid,
                                                int* lens_s, int* sel_s) {
  if (B > kThreads) return z;
  if (tid < B) lens_s[tid] = visible_end(p, tid);
  __syncthreads();
  if (tid < B) {
    const int li = lens_s[tid];
    int rank = 0;
    for (int j = 0; j < B; ++j) {
      const int lj = lens_s[j];
      rank += (lj > li) || (lj == li && j < tid);
    }
    if (rank == z) *sel_s = tid;   // ranks are a permutation of 0 .. B - 1
  }
  __syncthreads();
  return *sel_s;
}

// Rows [k0, k0 + rows) of cache head (b, g), k0 a multiple of 64 (and rows <= 64 in
// paged mode, so the rows lie in one page).  `valid` counts the rows below hi that
// are backed by memory; a page index outside [0, n_pages) backs none, so its keys
// are never read and are treated as invisible.
struct KvSpan {
  const uint16_t* k;
  const uint16_t* v;
  int valid;
};
template <int D>
__device__ __forceinline__ KvSpan kv_span(const DecodeParams& p, int b, int g, int k0, int rows, int hi) {
  int valid = max(0, min(rows, hi - k0));
  size_t off = 0;
  if (valid > 0) {
    if (p.block_table) {
      const int pg = p.block_table[(size_t)b * p.max_pages + k0 / p.page_size];
      if (pg >= 0 && pg < p.n_pages) off = (((size_t)pg * p.h_kv + g) * p.page_size + k0 % p.page_size) * D;
      else valid = 0;
    } else {
      off = ((size_t)(b * p.h_kv + g) * p.T_cap + k0) * D;
    }
  }
  return KvSpan{p.k + off, p.v + off, valid};
}

template <int D, bool OUT_BF16, bool ROPE>
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
  __shared__ int lens_s[kThreads];
  __shared__ int sel_s;
  const int b = sequence_of_rank(p, blockIdx.z, gridDim.z, tid, lens_s, &sel_s);

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
    if constexpr (ROPE) {
      // qf[ks] and qf[ks + D/32] hold elements 16 ks + 8 h + e and their partners
      const int qp = query_position(p, b);
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        uint64_t th[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) th[e] = h ? p.rope_theta.t[16 * ks + 8 + e] : p.rope_theta.t[16 * ks + e];
        rope_rotate8(qf[ks], qf[ks + D / 32], qp, th);
      }
    }
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // a 128-key tile is two 64-row halves, each read through its own descriptor whose
  // range ends at the half's last backed row (reads past it return zeros)
  constexpr int UNITS = kTile * D / 8 / kThreads;           // 16-byte chunks per thread per tensor
  uint4 kreg[UNITS], vreg[UNITS];
  int lim_next[2], lim_cur[2];
  auto load_tile = [&](int k0) {
    const KvSpan s0 = kv_span<D>(p, b, g, k0, 64, hi);
    const KvSpan s1 = kv_span<D>(p, b, g, k0 + 64, 64, hi);
    const __amdgpu_buffer_rsrc_t kr0 = make_rsrc(s0.k, (uint32_t)s0.valid * D * 2);
    const __amdgpu_buffer_rsrc_t vr0 = make_rsrc(s0.v, (uint32_t)s0.valid * D * 2);
    const __amdgpu_buffer_rsrc_t kr1 = make_rsrc(s1.k, (uint32_t)s1.valid * D * 2);
    const __amdgpu_buffer_rsrc_t vr1 = make_rsrc(s1.v, (uint32_t)s1.valid * D * 2);
    lim_next[0] = k0 + s0.valid;
    lim_next[1] = k0 + 64 + s1.valid;
#pragma unroll
    for (int i = 0; i < UNITS; ++i) {
      const int u = tid + kThreads * i;
      const int row = u / (D / 8), c8 = u % (D / 8);
      const bool second = i >= UNITS / 2;                     // rows 64..127 (uniform per i)
      const uint32_t off = (uint32_t)((row - (second ? 64 : 0)) * D + c8 * 8) * 2;
      kreg[i] = load16(second ? kr1 : kr0, off);
      vreg[i] = load16(second ? vr1 : vr0, off);
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
    lim_cur[0] = lim_next[0];
    lim_cur[1] = lim_next[1];
    if (t + 1 < n_tiles) load_tile(k0 + kTile);
    lds_barrier();                 // tile t is in LDS

    const unsigned char* vs_ = lds + L::K_BYTES;
    const int kw = wave * 32;      // this wave's 32-key block of the tile
    const int lim = lim_cur[wave >> 1];   // keys at or past lim are invisible
    f32x16 sacc;
#pragma unroll
    for (int kd = 0; kd < D / 16; ++kd) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds + (kw + col) * L::KS + (kd * 16 + h * 8) * 2);
      sacc = mfma32(a, qf[kd], kd == 0 ? f32x16{} : sacc);
    }
    if (k0 + kw + 32 > lim) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + kw + 8 * (e >> 2) + 4 * h + (e & 3);
        sacc[e] = key < lim ? sacc[e] : -INFINITY;
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
  constexpr int MS = merge_stride<D>();
  float* mo = reinterpret_cast<float*>(lds);              // [wave][32][MS]
  float* mml = mo + 4 * 32 * MS;                           // [wave][32][2]
  const float l_pair = pair_sum(l_run);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int d = db * 32 + 8 * e4 + 4 * h;
      *reinterpret_cast<float4*>(mo + (wave * 32 + col) * MS + d) =
          make_float4(oacc[db][4 * e4], oacc[db][4 * e4 + 1], oacc[db][4 * e4 + 2], oacc[db][4 * e4 + 3]);
    }
  if (h == 0) {
    mml[(wave * 32 + col) * 2 + 0] = (m_run == -INFINITY) ? -INFINITY : m_run * p.c;
    mml[(wave * 32 + col) * 2 + 1] = l_pair;
  }
  lds_barrier();
  merge_and_store<D, 32, OUT_BF16>(p, mo, mml, b, g * p.r + hcix * 32, n_heads_here, split, tid);
}

// ---------------------------------------------------------------------------
// Narrow groups (r <= 16): 16x16 matrix-core tiles.
//   S^T (16 keys x 16 heads) = K Q^T   v_mfma_f32_16x16x32_bf16, reduction over d_h
//     A: lane l holds K[key l%16][d = 32 kd + 8 (l/16) .. +7]   (16 bytes from LDS)
//     B: lane l holds Q[head l%16][same d]                        (registers)
//     C: lane l, element i holds S^T[key 4 (l/16) + i][head l%16]
//   O^T (16 d x 16 heads) += V^T P^T   v_mfma_f32_16x16x16_bf16, reduction over 16 keys
//     A: lane l holds V[key 4 (l/16) + t][d = 16 dt + l%16], t = 0..3: one transposing
//        LDS read (16-lane group G reads keys 4G..4G+3 of d 16 dt .. 16 dt + 15)
//     B: lane l holds P[head l%16][key 4 (l/16) + t]: the S^T accumulator itself
// A head's 16 keys of a block sit in the four lanes l%16 + 16 {0,1,2,3}, so its
// maximum and sum take one 16-lane and one 32-lane exchange.
constexpr int kTile16 = 64;         // keys per workgroup tile (16 per wave)

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float quad_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  return pair_max(x);
}
__device__ __forceinline__ float quad_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  return pair_sum(x);
}

template <int D>
struct Decode16Lds {
  static constexpr int KS = D * 2 + 16;
  static constexpr int VS = D * 2 + 32;
  static constexpr int K_BYTES = kTile16 * KS;
  static constexpr int STAGE = K_BYTES + kTile16 * VS;
  static constexpr int MERGE = merge_bytes<D, 16>();
  static constexpr int TOTAL = STAGE > MERGE ? STAGE : MERGE;
};

template <int D, bool OUT_BF16, bool ROPE>
__global__ void __launch_bounds__(kThreads, 4)
decode16_bf16_kernel(DecodeParams p) {
  using L = Decode16Lds<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int q16 = lane & 15;      // query head of the group held by this lane
  const int G = lane >> 4;        // lane group: keys 4G .. 4G+3 of a 16-key block

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  __shared__ int lens_s[kThreads];
  __shared__ int sel_s;
  const int b = sequence_of_rank(p, blockIdx.z, gridDim.z, tid, lens_s, &sel_s);

  // split s takes tiles s, s + n_split, s + 2 n_split, ... of the history, so the
  // workgroups of one sequence stream neighbouring memory at the same time
  const int kv_end = visible_end(p, b);
  const int n_all = (kv_end + kTile16 - 1) / kTile16;
  const int n_tiles = n_all > split ? (n_all - split + p.n_split - 1) / p.n_split : 0;
  const int hi = kv_end;
  const int n_heads_here = p.r;   // <= 16

  // fused append: position wp of (b, g) takes the new row.  Only the split whose
  // tiles hold wp reads that row, and it takes the new values in place of the
  // cache's (below, in load_tile); the same split writes the row to the cache
  // (split 0 when no split reads it).  A position outside the cache, or on a page
  // outside the pool, is skipped, as by kv_append.
  int wp = -1;
  if (p.write_pos) {
    wp = p.write_pos[b];
    const int cap = p.block_table ? p.max_pages * p.page_size : p.T_cap;
    if (wp < 0 || wp >= cap) wp = -1;
  }
  if (wp >= 0) {
    const int tw = wp / kTile16;
    if (split == (tw < n_all ? tw % p.n_split : 0) && tid < D / 4) {
      size_t row = ((size_t)(b * p.h_kv + g) * p.T_cap + wp) * D;
      bool backed = true;
      if (p.block_table) {
        const int pg = p.block_table[(size_t)b * p.max_pages + wp / p.page_size];
        backed = pg >= 0 && pg < p.n_pages;
        row = (((size_t)pg * p.h_kv + g) * p.page_size + wp % p.page_size) * D;
      }
      if (backed) {
        const int c8 = tid % (D / 8);
        const size_t src = (size_t)(b * p.h_kv + g) * D + c8 * 8;
        // the caches are the caller's writable buffers; only this path writes them
        if (tid < D / 8)
          *reinterpret_cast<uint4*>(const_cast<uint16_t*>(p.k) + row + c8 * 8) = new_key_chunk<D, ROPE>(p, b, g, c8, wp);
        else
          *reinterpret_cast<uint4*>(const_cast<uint16_t*>(p.v) + row + c8 * 8) =
              *reinterpret_cast<const uint4*>(p.v_new + src);
      }
    }
  }

  if (n_tiles == 0) {
    if (p.direct) {
      for (int e = tid; e < n_heads_here * D; e += kThreads) {
        const int j = e / D, d = e % D;
        const size_t oi = (size_t)(b * p.h_q + g * p.r + j) * D + d;
        if constexpr (OUT_BF16) static_cast<uint16_t*>(p.o)[oi] = 0;
        else static_cast<float*>(p.o)[oi] = 0.f;
      }
    }
    return;
  }

  const bool q_valid = q16 < n_heads_here;
  bf16x8 qf[D / 32];
  {
    const uint16_t* qrow = p.q + (size_t)(b * p.h_q + g * p.r + q16) * D;
#pragma unroll
    for (int kd = 0; kd < D / 32; ++kd) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (q_valid) x = *reinterpret_cast<const uint4*>(qrow + kd * 32 + G * 8);
      qf[kd] = __builtin_bit_cast(bf16x8, x);
    }
    if constexpr (ROPE) {
      // qf[kd] and qf[kd + D/64] hold elements 32 kd + 8 G + e and their partners
      const int qp = query_position(p, b);
#pragma unroll
      for (int kd = 0; kd < D / 64; ++kd) {
        uint64_t th[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint64_t* t = p.rope_theta.t + 32 * kd + e;
          th[e] = G == 0 ? t[0] : G == 1 ? t[8] : G == 2 ? t[16] : t[24];
        }
        rope_rotate8(qf[kd], qf[kd + D / 64], qp, th);
      }
    }
  }

  f32x4 oacc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // each 64-key tile is read through its own descriptor whose range ends at the
  // tile's last backed row (reads past it return zeros)
  constexpr int UNITS = kTile16 * D / 8 / kThreads;
  uint4 kreg[UNITS], vreg[UNITS];
  int lim_next = 0, lim_cur = 0;
  auto load_tile = [&](int k0) {
    const KvSpan sp = kv_span<D>(p, b, g, k0, kTile16, hi);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(sp.k, (uint32_t)sp.valid * D * 2);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(sp.v, (uint32_t)sp.valid * D * 2);
    lim_next = k0 + sp.valid;
#pragma unroll
    for (int i = 0; i < UNITS; ++i) {
      const int u = tid + kThreads * i;
      const int row = u / (D / 8), c8 = u % (D / 8);
      const uint32_t off = (uint32_t)(row * D + c8 * 8) * 2;
      kreg[i] = load16(krs, off);
      vreg[i] = load16(vrs, off);
    }
    if (wp >= k0 && wp < k0 + kTile16) {
      // the appended row: new values in place of the cache's
#pragma unroll
      for (int i = 0; i < UNITS; ++i) {
        const int u = tid + kThreads * i;
        const int row = u / (D / 8), c8 = u % (D / 8);
        if (k0 + row == wp) {
          kreg[i] = new_key_chunk<D, ROPE>(p, b, g, c8, wp);
          vreg[i] = *reinterpret_cast<const uint4*>(p.v_new + (size_t)(b * p.h_kv + g) * D + c8 * 8);
        }
      }
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

  const int tstride = p.n_split * kTile16;
  load_tile(split * kTile16);
  for (int t = 0; t < n_tiles; ++t) {
    const int k0 = (split + t * p.n_split) * kTile16;
    lds_barrier();                 // every wave is done reading the previous tile
    store_tile();
    lim_cur = lim_next;            // keys at or past lim_cur are invisible
    if (t + 1 < n_tiles) load_tile(k0 + tstride);
    lds_barrier();                 // tile t is in LDS

    const unsigned char* vs_ = lds + L::K_BYTES;
    const int kw = wave * 16;      // this wave's 16 keys of the tile
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kd = 0; kd < D / 32; ++kd) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds + (kw + q16) * L::KS + (kd * 32 + G * 8) * 2);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[kd], sacc, 0, 0, 0);
    }
    if (k0 + kw + 16 > lim_cur) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + kw + 4 * G + i;
        sacc[i] = key < lim_cur ? sacc[i] : -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]));
    mx = quad_max(mx);
    const bool grow = (mx - m_run) * p.c > kLazyRescale;     // false for -inf - (-inf)
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? fast_exp2((m_run - mx) * p.c) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) oacc[dt] *= alpha;
      m_run = grow ? mx : m_run;
    }
    const float mc = (m_run == -INFINITY ? 0.f : m_run) * p.c;
    float pe[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pe[i] = fast_exp2(fmaf(sacc[i], p.c, -mc));
      l_run += pe[i];
    }
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 pb;
    pb[0] = (__bf16)pe[0]; pb[1] = (__bf16)pe[1]; pb[2] = (__bf16)pe[2]; pb[3] = (__bf16)pe[3];
    const s16x4 pf = __builtin_bit_cast(s16x4, pb);
    // V^T operand: source lane (j, q) of group G points at row kw + 4G + j, columns 16 dt + 4q
    const unsigned char* vsrc = vs_ + (kw + 4 * G + ((lane & 15) >> 2)) * L::VS + 4 * (lane & 3) * 2;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vsrc + dt * 32));
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pf, oacc[dt], 0, 0, 0);
    }
  }

  // ---- merge the 4 waves' states in LDS
  lds_barrier();
  constexpr int MS = merge_stride<D>();
  float* mo = reinterpret_cast<float*>(lds);              // [wave][16][MS]
  float* mml = mo + 4 * 16 * MS;                           // [wave][16][2]
  const float l_all = quad_sum(l_run);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    *reinterpret_cast<float4*>(mo + (wave * 16 + q16) * MS + dt * 16 + 4 * G) =
        make_float4(oacc[dt][0], oacc[dt][1], oacc[dt][2], oacc[dt][3]);
  if (G == 0) {
    mml[(wave * 16 + q16) * 2 + 0] = (m_run == -INFINITY) ? -INFINITY : m_run * p.c;
    mml[(wave * 16 + q16) * 2 + 1] = l_all;
  }
  lds_barrier();
  merge_and_store<D, 16, OUT_BF16>(p, mo, mml, b, g * p.r, n_heads_here, split, tid);
}

// Merge the partial states of one (sequence, query head): [AttnVar] 3.5 applied
// split after split.  Four waves per output row each fold every fourth split,
// then the four states are folded in LDS.
template <int D, bool OUT_BF16>
__global__ void __launch_bounds__(256)
decode_combine_kernel(DecodeParams p) {
  __shared__ float st_u[4][D];
  __shared__ float st_ml[4][2];
  const int head = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kv_end = visible_end(p, b);
  // live splits: contiguous slices of `chunk` keys, or (interleaved) one tile each round
  const int n = p.interleave ? min(p.n_split, (kv_end + kTile16 - 1) / kTile16)
                             : (kv_end + p.chunk - 1) / p.chunk;
  const size_t base = (size_t)(b * p.h_q + head) * p.n_split_cap;
  constexpr int PER = D / 64;
  float M = -INFINITY, Lsum = 0.f, U[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) U[i] = 0.f;
  for (int s = wave; s < n; s += 4) {
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
#pragma unroll
  for (int i = 0; i < PER; ++i) st_u[wave][lane + 64 * i] = U[i];
  if (lane == 0) { st_ml[wave][0] = M; st_ml[wave][1] = Lsum; }
  __syncthreads();
  if (wave != 0) return;
  float Mt = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) Mt = fmaxf(Mt, st_ml[w][0]);
  float wgt[4], Lt = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wgt[w] = st_ml[w][0] == -INFINITY ? 0.f : fast_exp2(st_ml[w][0] - Mt);
    Lt += wgt[w] * st_ml[w][1];
  }
  const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    float u = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) u += wgt[w] * st_u[w][lane + 64 * i];
    const size_t oi = (size_t)(b * p.h_q + head) * D + lane + 64 * i;
    if constexpr (OUT_BF16) {
      __bf16 x = (__bf16)(u * inv);
      static_cast<uint16_t*>(p.o)[oi] = __builtin_bit_cast(uint16_t, x);
    } else {
      static_cast<float*>(p.o)[oi] = u * inv;
    }
  }
}

// The same merge for many splits (more than kManySplits): thread (split lane j,
// unit q) folds splits j, j + NJ, j + 2 NJ, ... for d = 4q .. 4q + 3, with the
// states of eight of its splits requested at once instead of one split after
// another; the NJ states of a unit are then folded in LDS in split-lane order.
template <int D, bool OUT_BF16>
__global__ void __launch_bounds__(256)
decode_combine_many_kernel(DecodeParams p) {
  constexpr int Q = D / 4;             // 4-wide units of d
  constexpr int NJ = 256 / Q;          // split lanes
  __shared__ float4 st_u[NJ][Q];
  __shared__ float2 st_ml[NJ][Q];
  const int head = blockIdx.x;
  const int b = blockIdx.y;
  const int q = threadIdx.x % Q, j = threadIdx.x / Q;
  const int kv_end = visible_end(p, b);
  // live splits: contiguous slices of `chunk` keys, or (interleaved) one tile each round
  const int n = p.interleave ? min(p.n_split, (kv_end + kTile16 - 1) / kTile16)
                             : (kv_end + p.chunk - 1) / p.chunk;
  const size_t base = (size_t)(b * p.h_q + head) * p.n_split_cap;
  auto fold = [](float& M, float& L, float4& U, float ms, float ls, float4 us) {
    if (ms == -INFINITY) return;
    const float Mn = fmaxf(M, ms);
    const float a = fast_exp2(M - Mn);       // 0 on the first live state
    const float w = fast_exp2(ms - Mn);
    L = a * L + w * ls;
    U = make_float4(a * U.x + w * us.x, a * U.y + w * us.y, a * U.z + w * us.z, a * U.w + w * us.w);
    M = Mn;
  };
  float M = -INFINITY, L = 0.f;
  float4 U = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = j; s0 < n; s0 += 8 * NJ) {
    float ms[8], ls[8];
    float4 us[8];
    // unconditional loads (a split past n re-reads split n - 1 and is dropped) keep
    // all eight requests in flight together
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int sp = min(s0 + k * NJ, n - 1);
      const float2 ml = *reinterpret_cast<const float2*>(p.ws_ml + (base + sp) * 2);
      ms[k] = s0 + k * NJ < n ? ml.x : -INFINITY;
      ls[k] = ml.y;
      us[k] = *reinterpret_cast<const float4*>(p.ws_u + (base + sp) * D + 4 * q);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) fold(M, L, U, ms[k], ls[k], us[k]);
  }
  st_u[j][q] = U;
  st_ml[j][q] = make_float2(M, L);
  __syncthreads();
  if (j != 0) return;
  float Mt = -INFINITY, Lt = 0.f;
  float4 Ut = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) fold(Mt, Lt, Ut, st_ml[jj][q].x, st_ml[jj][q].y, st_u[jj][q]);
  const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
  const size_t oi = (size_t)(b * p.h_q + head) * D + 4 * q;
  if constexpr (OUT_BF16) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 w4;
    w4[0] = (__bf16)(Ut.x * inv); w4[1] = (__bf16)(Ut.y * inv); w4[2] = (__bf16)(Ut.z * inv); w4[3] = (__bf16)(Ut.w * inv);
    *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(p.o) + oi) = w4;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(p.o) + oi) = make_float4(Ut.x * inv, Ut.y * inv, Ut.z * inv, Ut.w * inv);
  }
}

template <int D, bool OUT_BF16, bool ROPE>
hipError_t launch_split(const DecodeParams& prm, int B, hipStream_t s) {
  if (prm.r <= 16) {
    constexpr int smem = Decode16Lds<D>::TOTAL;
    static std::atomic<unsigned long long> lds_allowed{0};
    const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(decode16_bf16_kernel<D, OUT_BF16, ROPE>),
                                           smem, lds_allowed);
    if (e != hipSuccess) return e;
    dim3 grid(prm.n_split, prm.h_kv, B);
    hipLaunchKernelGGL((decode16_bf16_kernel<D, OUT_BF16, ROPE>), grid, dim3(kThreads), smem, s, prm);
  } else {
    constexpr int smem = DecodeLds<D>::TOTAL;
    static std::atomic<unsigned long long> lds_allowed{0};
    const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(decode_bf16_kernel<D, OUT_BF16, ROPE>),
                                           smem, lds_allowed);
    if (e != hipSuccess) return e;
    dim3 grid(prm.n_split, prm.h_kv * prm.hc_count, B);
    hipLaunchKernelGGL((decode_bf16_kernel<D, OUT_BF16, ROPE>), grid, dim3(kThreads), smem, s, prm);
  }
  return hipGetLastError();
}

template <int D, bool OUT_BF16>
hipError_t launch_t(const DecodeParams& prm, int B, hipStream_t s) {
  hipError_t e = prm.rope ? launch_split<D, OUT_BF16, true>(prm, B, s) : launch_split<D, OUT_BF16, false>(prm, B, s);
  if (e != hipSuccess || prm.direct) return e;
  if (prm.n_split > kManySplits)
    hipLaunchKernelGGL((decode_combine_many_kernel<D, OUT_BF16>), dim3(prm.h_q, B), dim3(256), 0, s, prm);
  else
    hipLaunchKernelGGL((decode_combine_kernel<D, OUT_BF16>), dim3(prm.h_q, B), dim3(256), 0, s, prm);
  return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode_bf16(int B, int h_q, int h_kv, int T_cap, int D, int len) {
  DecodePlan pl;
  const int r = h_q / h_kv;
  const bool narrow = r <= 16;            // 16x16 tiles, 4 workgroups per CU
  pl.head_chunks = narrow ? 1 : (r + 31) / 32;
  const long long pairs = (long long)B * h_kv * pl.head_chunks;
  const long long target = narrow ? 4 * kTargetWG : kTargetWG;
  long long cap = (target + pairs - 1) / pairs;
  if (cap < 1) cap = 1;
  const long long max_cap = (T_cap + kMinChunk - 1) / kMinChunk;
  if (cap > max_cap) cap = max_cap < 1 ? 1 : max_cap;
  // The 16x16 kernel streams short slices less well: halve the split count while a
  // full-length slice is under kPreferChunk keys and kTargetWG workgroups remain
  // (B=8, h_kv=8, T=32000: 8 splits of 4000 keys ran 5% faster than 16 of 2000).
  // Only T_cap enters, so the workspace sized for T_cap fits every call.  The 16x16
  // kernel's larger target pays on ragged batches: B=32, h_kv=8, lengths uniform on
  // 1..32768, 8 splits per sequence in longest-first order ran 9% faster than 4.
  if (narrow)
    while (cap > 1 && (T_cap + cap - 1) / cap < kPreferChunk && pairs * (cap / 2) >= kTargetWG) cap /= 2;
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
  if (a.write_pos && a.h_q / a.h_kv > 16) return hipErrorInvalidValue;   // fused append: 16x16 kernel only
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
  p.interleave = p.r <= 16 ? 1 : 0;
  p.block_table = a.block_table;
  p.page_size = a.page_size; p.max_pages = a.max_pages; p.n_pages = a.n_pages;
  p.k_new = static_cast<const uint16_t*>(a.k_new);
  p.v_new = static_cast<const uint16_t*>(a.v_new);
  p.write_pos = a.write_pos;
  p.c = a.scale * kLog2e;
  p.rope = a.rope_base > 0.f ? 1 : 0;
  p.rope_theta = p.rope ? make_rope_theta(a.D, a.rope_base) : RopeTheta{};
  const size_t u_bytes = (size_t)a.B * a.h_q * pl.n_split_cap * a.D * sizeof(float);
  p.ws_u = static_cast<float*>(a.workspace);
  p.ws_ml = a.workspace ? reinterpret_cast<float*>(static_cast<char*>(a.workspace) + u_bytes) : nullptr;
  if (a.D == 128) return a.out_bf16 ? launch_t<128, true>(p, a.B, s) : launch_t<128, false>(p, a.B, s);
  return a.out_bf16 ? launch_t<64, true>(p, a.B, s) : launch_t<64, false>(p, a.B, s);
}

}  // namespace gqa
