// bf16 grouped-query attention on the gfx950 matrix cores: prefill and
// chunked prefill, head width 64 or 128, fp32 accumulation.
//
// Method ([EffSeq] 分块注意力 and 在线 softmax; [AttnVar] 3.5): the score and
// probability matrices are never written to memory.  A workgroup owns 256
// query rows of one (sequence b, K/V head g) and walks the keys in 64-key
// tiles.  Each K tile and V tile is loaded from HBM once per workgroup into
// LDS and serves every query head of the group that the workgroup holds
// ([MhaMqaGqa] section 7: one K/V tile serves all r query rows of its group;
// rows are positions x heads and keep their own causal position); its 8 waves
// take 32 rows each, so one staged tile feeds 256 rows.  Per tile, every wave
// computes
//     S^T = K Q^T                (matrix core, reduction over d_h)
//     m'  = max(m, rowmax S)     (lane-local plus one lane-pair exchange; m is only
//                                 moved when the tile maximum exceeds it by more
//                                 than 2^kLazyRescale, so most tiles skip the rescale)
//     P   = exp2(S c - m' c),  c = scale * log2(e)
//     l   = e^{m - m'} l + rowsum P,   O^T = e^{m - m'} O^T + V^T P^T   (matrix core)
// and after the last tile writes O = O^T / l.  Keys a row cannot see are
// removed by selection before the maximum; tiles past the causal frontier
// are never visited; a row that sees no key is written as zeros.
//
// Layouts in LDS (two stages, double-buffered), both filled by 16-byte buffer
// loads that return zeros past the last visible key (no per-load branches):
//   K [64 keys][d_h] row-major, rows padded by 8 bytes; the K operand is read as two
//     8-byte halves, conflict-free at this stride
//   V [64 keys][d_h] row-major, rows padded by 32 bytes (conflict-free transposing
//     reads, which hand the PV product its V^T operand directly).
#include "internal.h"
#include "mfma_common.h"

namespace gqa {
namespace {

constexpr int kThreads = 512;   // 8 waves, 2 per SIMD
constexpr int kRowsWG = 256;    // query rows per workgroup (32 per wave)
constexpr int kTile = 64;       // keys per tile

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  const int32_t* kv_lens;
  const int32_t* q_pos0;
  int h_q, h_kv, r, hp, P;      // hp heads x P positions = 256 rows per workgroup
  int S_q, T_cap;
  int causal, from_end;
  int n_qblocks, n_hchunks;
  int xcd_remap;
  float c;                      // scale * log2(e)
};

template <int D>
struct PrefillLds {
  static constexpr int KS = D * 2 + 8;           // K row stride, bytes (8-byte reads conflict-free)
  static constexpr int VS = D * 2 + 32;          // V row stride, bytes
  static constexpr int K_BYTES = kTile * KS;
  static constexpr int STAGE = K_BYTES + kTile * VS;
  static constexpr int TOTAL = 2 * STAGE;
};

template <int D, bool OUT_BF16>
__global__ void __launch_bounds__(kThreads, 1)
prefill_bf16_kernel(PrefillParams p) {
  using L = PrefillLds<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;       // lane half
  const int col = lane & 31;     // query row within the wave

  // ---- work item: heaviest causal blocks first; blocks that share K/V stay on one XCD
  int vid = blockIdx.x;
  if (p.xcd_remap) vid = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int bgh = vid / p.n_qblocks;
  const int qb = p.n_qblocks - 1 - (vid % p.n_qblocks);
  const int hc = bgh % p.n_hchunks;
  const int bg = bgh / p.n_hchunks;
  const int g = bg % p.h_kv;
  const int b = bg / p.h_kv;

  const int len_b = clampi(p.kv_lens ? p.kv_lens[b] : p.T_cap, 0, p.T_cap);
  const int pos0 = p.q_pos0 ? p.q_pos0[b] : (p.from_end ? len_b - p.S_q : 0);

  // ---- this lane's query row
  const int rho = wave * 32 + col;
  const int hh = hc * p.hp + rho / p.P;
  const int qi = qb * p.P + rho % p.P;
  const bool row_valid = qi < p.S_q;
  const int head = g * p.r + hh;
  const int pos = pos0 + qi;

  // ---- key extent of the workgroup
  const int first_q = qb * p.P;
  const int last_q = min(first_q + p.P, p.S_q) - 1;
  int kv_end = len_b;
  if (p.causal) kv_end = min(len_b, max(pos0 + last_q + 1, 0));
  const int min_pos = pos0 + first_q;
  const int n_tiles = (kv_end + kTile - 1) / kTile;

  // ---- Q fragments (B operand of S^T = K Q^T), kept in registers
  bf16x8 qf[D / 16];
  {
    const uint16_t* qrow = p.q + ((size_t)(b * p.h_q + head) * p.S_q + qi) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (row_valid) x = *reinterpret_cast<const uint4*>(qrow + ks * 16 + h * 8);
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m_run = -INFINITY;   // unscaled running maximum of this row
  float l_run = 0.f;         // this lane's share of the normalizer

  const size_t kv_base = (size_t)(b * p.h_kv + g) * p.T_cap * D;
  const uint32_t slice_bytes = (uint32_t)kv_end * D * 2;     // keys >= kv_end read as zeros
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + kv_base, slice_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + kv_base, slice_bytes);

  // ---- tile loader: global -> registers -> LDS, 16 bytes per access
  constexpr int UNITS = kTile * D / 8 / kThreads;          // 16-byte chunks per thread per tensor
  uint4 kreg[UNITS], vreg[UNITS];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < UNITS; ++i) {
      const int u = tid + kThreads * i;
      const int row = u / (D / 8), c8 = u % (D / 8);
      const uint32_t off = (uint32_t)((t * kTile + row) * D + c8 * 8) * 2;
      kreg[i] = load16(krs, off);
      vreg[i] = load16(vrs, off);
    }
  };
  auto store_tile = [&](int stage) {
    unsigned char* ks_ = lds + stage * L::STAGE;
    unsigned char* vs_ = ks_ + L::K_BYTES;
#pragma unroll
    for (int i = 0; i < UNITS; ++i) {
      const int u = tid + kThreads * i;
      const int row = u / (D / 8), c8 = u % (D / 8);
      uint2* kd = reinterpret_cast<uint2*>(ks_ + row * L::KS + c8 * 16);   // rows are 8-byte aligned
      kd[0] = make_uint2(kreg[i].x, kreg[i].y);
      kd[1] = make_uint2(kreg[i].z, kreg[i].w);
      *reinterpret_cast<uint4*>(vs_ + row * L::VS + c8 * 16) = vreg[i];
    }
  };

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }

  for (int t = 0; t < n_tiles; ++t) {
    if (t + 1 < n_tiles) load_tile(t + 1);
    lds_barrier();

    const unsigned char* ks_ = lds + (t & 1) * L::STAGE;
    const unsigned char* vs_ = ks_ + L::K_BYTES;
    const int k0 = t * kTile;

    // S^T for the two 32-key halves of the tile
    f32x16 sacc[2];
#pragma unroll
    for (int kd = 0; kd < D / 16; ++kd) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = lds_read_bf16x8(ks_ + (kb * 32 + col) * L::KS + (kd * 16 + h * 8) * 2);
        sacc[kb] = mfma32(a, qf[kd], kd == 0 ? f32x16{} : sacc[kb]);
      }
    }
    // keep four K operand reads in flight ahead of the products that consume them
    sched_pipeline<D / 8, 2, 1, 4>();

    // mask only where some key of the tile may be invisible to some row
    const bool need_mask = (p.causal && k0 + kTile - 1 > min_pos) || (k0 + kTile > len_b);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + kb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
          const bool vis = key < len_b && (!p.causal || key <= pos);
          sacc[kb][e] = vis ? sacc[kb][e] : -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
    mx = pair_max(mx);
    // move the running maximum only when it grew by more than 2^kLazyRescale
    const bool grow = (mx - m_run) * p.c > kLazyRescale;     // false for -inf - (-inf)
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? fast_exp2((m_run - mx) * p.c) : 1.f;   // 0 on the first visible tile
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
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = fast_exp2(fmaf(sacc[kb][e], p.c, -mc));
        sacc[kb][e] = pe;
        psum += pe;
      }
    l_run += psum;

    // P^T fragments: chunk kc of the tile = elements 8*(kc&1) .. +7 of half kc>>1
    bf16x8 pf[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const f32x16& sv = sacc[kc >> 1];
      const int e0 = 8 * (kc & 1);
      pf[kc] = pack_bf16x8(sv[e0], sv[e0 + 1], sv[e0 + 2], sv[e0 + 3], sv[e0 + 4], sv[e0 + 5], sv[e0 + 6], sv[e0 + 7]);
    }
    // O^T += V^T P^T
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 a = load_vt_operand(vs_, L::VS, kc, db * 32, lane);
        oacc[db] = mfma32(a, pf[kc], oacc[db]);
      }
    sched_pipeline<4 * D / 32, 2, 1, 4>();

    if (t + 1 < n_tiles) store_tile((t + 1) & 1);
  }

  // ---- epilogue: o = u / l
  const float l_tot = pair_sum(l_run);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (row_valid) {
    const size_t obase = ((size_t)(b * p.h_q + head) * p.S_q + qi) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = db * 32 + 8 * j + 4 * h;
        const float o0 = oacc[db][4 * j] * inv, o1 = oacc[db][4 * j + 1] * inv;
        const float o2 = oacc[db][4 * j + 2] * inv, o3 = oacc[db][4 * j + 3] * inv;
        if constexpr (OUT_BF16) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 w;
          w[0] = (__bf16)o0; w[1] = (__bf16)o1; w[2] = (__bf16)o2; w[3] = (__bf16)o3;
          *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(p.o) + obase + d0) = w;
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(p.o) + obase + d0) = make_float4(o0, o1, o2, o3);
        }
      }
  }
}

template <int D, bool OUT_BF16>
hipError_t launch_t(const PrefillParams& prm, int total, hipStream_t s) {
  constexpr int smem = PrefillLds<D>::TOTAL;
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(prefill_bf16_kernel<D, OUT_BF16>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL((prefill_bf16_kernel<D, OUT_BF16>), dim3(total), dim3(kThreads), smem, s, prm);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
  PrefillParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = a.o;
  p.kv_lens = a.kv_lens;
  p.q_pos0 = a.q_pos0;
  p.h_q = a.h_q; p.h_kv = a.h_kv; p.r = a.h_q / a.h_kv;
  // heads of one group per workgroup: the largest power of two dividing r, at most 128
  int hp = 1;
  while (hp < kRowsWG && p.r % (hp * 2) == 0) hp *= 2;
  p.hp = hp;
  p.P = kRowsWG / hp;
  p.S_q = a.S_q; p.T_cap = a.T_cap;
  p.causal = a.causal; p.from_end = a.q_pos_from_end;
  p.n_qblocks = (a.S_q + p.P - 1) / p.P;
  p.n_hchunks = p.r / hp;
  p.c = a.scale * kLog2e;
  const long long total = (long long)a.B * a.h_kv * p.n_hchunks * p.n_qblocks;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  p.xcd_remap = (total % 8 == 0) ? 1 : 0;
  if (a.D == 128) return a.out_bf16 ? launch_t<128, true>(p, (int)total, s) : launch_t<128, false>(p, (int)total, s);
  return a.out_bf16 ? launch_t<64, true>(p, (int)total, s) : launch_t<64, false>(p, (int)total, s);
}

}  // namespace gqa
