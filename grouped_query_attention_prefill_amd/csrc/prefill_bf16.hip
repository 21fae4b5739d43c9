// bf16 grouped-query attention on the gfx950 matrix cores: prefill and
// chunked prefill, head width 64 or 128, fp32 accumulation.
//
// Method ([EffSeq] 分块注意力 and 在线 softmax; [AttnVar] 3.5): the score and
// probability matrices are never written to memory.  A workgroup owns 256
// query rows of one (sequence b, K/V head g) and walks the keys in 128-key
// tiles.  Each K tile and V tile is loaded from memory once per workgroup into
// LDS and serves every query head of the group that the workgroup holds
// ([MhaMqaGqa] section 7: one K/V tile serves all r query rows of its group;
// rows are positions x heads and keep their own causal position); its 8 waves
// take 32 rows each, so one staged tile feeds 256 rows.  Per tile t, every wave
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
// Schedule: the work of a tile is split into a matrix phase (O^T += V^T P^T for
// the previous tile, then S^T = K Q^T for this one) and a vector phase (mask,
// maximum, exponentials, row sums, P packed to bf16 in the score registers).  The
// 8 waves form two groups of four, one wave of each on every SIMD, and the second
// group runs one phase behind the first: while one wave of a SIMD keeps the matrix
// core busy, the other does its exponentials, and a workgroup barrier between
// phases keeps the two groups in step.  The trailing group stages the tiles: during
// its vector phase, while the leading group's matrix phase t runs, it requests K
// tile t + 1 and V tile t with buffer loads that write LDS directly (no registers
// pass them), each wave at its own point of the phase, and it waits for them at the
// end of its next matrix phase, before their first reader; the leading group's
// matrix phases carry no load instructions.  The ROPE instances rotate the
// workgroup's Q rows at their positions (in LDS, before any tile is loaded).  O is
// written through LDS as whole 128-byte lines with the non-temporal hint.
//
// Layouts in LDS, filled 1 KiB per load instruction (64 lanes x 16 bytes); keys
// past the last visible one read as zeros (the buffer range ends there):
//   K [128 keys][d_h] row-major, rows padded by 16 bytes: 16-byte operand reads
//     are conflict-free at this stride (at 32 bytes of padding they take twice
//     the cycles)
//   V [128 keys][d_h] row-major, rows padded by 32 bytes, read with transposing
//     reads that hand the PV product its V^T operand directly (rows of 256 or
//     272 bytes made the launch 6% and 5.5% slower).
#include <type_traits>

#include "internal.h"
#include "mfma_common.h"
#include "rope_common.h"

namespace gqa {
namespace {

constexpr int kThreads = 512;   // 8 waves: two groups of 4, one wave of each per SIMD
constexpr int kGroup = 256;     // threads per group
constexpr int kRowsWG = 256;    // query rows per workgroup (32 per wave)
constexpr int kTile = 128;      // keys per tile

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;                   // (B, h_q, S_q) row log-sum-exp, or null
  const int32_t* kv_lens;
  const int32_t* q_pos0;
  int h_q, h_kv, r, hp, P;      // hp heads x P positions = 256 rows per workgroup
  int S_q, T_cap;
  int causal, from_end;
  int n_qblocks, n_hchunks;
  int xcd_remap;
  float c;                      // scale * log2(e)
  float scale;
  int rope;                     // rotate Q at each row's position as it is loaded (the ROPE kernels)
  RopeTheta rope_theta;
};

// LDS: two K stages, then two V stages, each a 128-key tile with padded rows.  The
// stages are filled by buffer loads that write LDS directly, 1 KiB per instruction
// (64 lanes x 16 bytes, lane i at byte 16 i); a lane whose 16 bytes fall in a row's
// padding reads outside its descriptor's range, so it touches no memory and writes
// zeros into padding that no product reads.
template <int D>
struct PrefillLds {
  static constexpr int KS = D * 2 + 16;          // K row stride, bytes
  static constexpr int VS = D * 2 + 32;          // V row stride, bytes
  static constexpr int K_STAGE = kTile * KS;
  static constexpr int V_STAGE = kTile * VS;
  static constexpr int V_OFF = 2 * K_STAGE;      // two K stages, then two V stages
  static constexpr int TOTAL = 2 * K_STAGE + 2 * V_STAGE;
  static constexpr int K_BLOCKS = K_STAGE / 1024;
  static constexpr int V_BLOCKS = V_STAGE / 1024;
  static constexpr int MAXB = (V_BLOCKS + 3) / 4; // 1 KiB blocks per wave and tile (four waves per group)
  static_assert(K_STAGE % 1024 == 0 && V_STAGE % 1024 == 0, "stages are whole 1 KiB blocks");
  static_assert(V_BLOCKS >= K_BLOCKS, "the V stage is the larger");
  static_assert(TOTAL <= 160 * 1024, "fits the LDS of one CU");
};

// One 16-byte-per-lane buffer load written straight into LDS: lane i's 16 bytes from
// byte voff + soff of the descriptor's range land at dst + 16 i (dst wave-uniform).
// A plain device function, so that only the device compilation sees the LDS pointer.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, unsigned char* dst, uint32_t voff,
                                           uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}

// s_waitcnt vmcnt(0): the buffer loads that write LDS are counted only by vmcnt; the
// loading waves wait for them explicitly, at the end of the phase before the one that
// reads the stage, and the next stage_barrier hands the stage to the other waves.
__device__ __forceinline__ void wait_lds_loads() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier between phases: this wave's LDS reads and writes are complete
// (lgkmcnt(0)); no memory access is moved across it by the compiler (the empty asm
// statements clobber memory) and no instruction by its scheduler (sched_barrier), so
// each phase's work stays on its side.  Unlike a release fence, it does not wait for
// the tile loads still in flight into LDS, which are waited for by wait_lds_loads.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt not waited for
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier after a vector phase: that phase reads and writes no LDS, so no
// wait precedes the barrier (the same compiler and scheduler fences as above).
__device__ __forceinline__ void vector_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Products of one matrix phase in issue order.  QK product (kb, kd): S^T block kb (32
// keys) += K-chunk x Q-chunk kd (16 values of d); PV product (kc, db): O^T block db (32
// values of d) += V^T x P^T over 16-key chunk kc.  P^T of chunk kc lives in the first
// half of the score registers of block kc / 2, so the PV products of chunks 2 kb and
// 2 kb + 1 come before the QK product that overwrites block kb; consecutive products
// never write the same accumulator.
template <int D, bool QK, bool PV>
struct PhaseOrder {
  static constexpr int NKD = D / 16;             // QK products per key block
  static constexpr int NDB = D / 32;             // PV products per key chunk
  static constexpr int SEG = 2 * NDB;            // == NKD
  static constexpr int N = (QK ? 4 * NKD : 0) + (PV ? 8 * NDB : 0);
  // returns pv * 256 + x * 16 + y with (x, y) = (kc, db) or (kb, kd)
  static constexpr int at(int j) {
    if (QK && PV) {
      if (j < SEG) return 256 + (j / NDB) * 16 + j % NDB;
      if (j < 3 * SEG) {
        const int m = j - SEG;
        return (m & 1) ? 256 + (2 + (m / 2) / NDB) * 16 + (m / 2) % NDB : 0 * 16 + m / 2;
      }
      if (j < 5 * SEG) {
        const int m = j - 3 * SEG;
        return (m & 1) ? 256 + (4 + (m / 2) / NDB) * 16 + (m / 2) % NDB : 1 * 16 + m / 2;
      }
      if (j < 6 * SEG) return 256 + (6 + (j - 5 * SEG) / NDB) * 16 + (j - 5 * SEG) % NDB;
      const int m = j - 6 * SEG;
      return (2 + (m & 1)) * 16 + m / 2;
    }
    if (QK) return (2 * (j / (2 * NKD)) + (j & 1)) * 16 + (j % (2 * NKD)) / 2;
    return 256 + (j / NDB) * 16 + j % NDB;
  }
};

template <int D, bool OUT_BF16, bool ROPE>
__global__ void __launch_bounds__(kThreads, 1)
prefill_bf16_kernel(PrefillParams p) {
  using L = PrefillLds<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;     // 0: leads, stages K; 1: one phase behind, stages V
  const int gw = wave & 3;       // wave within the group
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
  bf16x8 qf[D / 16] = {};
  if constexpr (!ROPE) {
    const uint16_t* qrow = p.q + ((size_t)(b * p.h_q + head) * p.S_q + qi) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (row_valid) x = *reinterpret_cast<const uint4*>(qrow + ks * 16 + h * 8);
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }
  // Rotary encoding at each row's absolute position, applied to the workgroup's Q
  // rows staged in LDS before any tile is loaded: wave w turns the pairs 8 w .. 8 w + 7
  // of rows lane + 64 k, so its angles are wave-uniform; then every lane reads its
  // fragments as above.
  auto load_q_rotated = [&]() {
    constexpr int QS = D * 2 + 16;                       // row stride, bytes (<= the K/V stages)
    constexpr int CH = D / 8;                            // 16-byte chunks per row
    static_assert(kRowsWG * QS <= PrefillLds<D>::TOTAL, "Q rows fit the stage space");
#pragma unroll
    for (int j = 0; j < kRowsWG * CH / kThreads; ++j) {
      const int u = tid + kThreads * j;
      const int r_ = u / CH, c_ = u % CH;
      const int hh_ = hc * p.hp + r_ / p.P, qi_ = qb * p.P + r_ % p.P;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (qi_ < p.S_q)
        x = *reinterpret_cast<const uint4*>(p.q + ((size_t)(b * p.h_q + g * p.r + hh_) * p.S_q + qi_) * D + c_ * 8);
      *reinterpret_cast<uint4*>(lds + r_ * QS + c_ * 16) = x;
    }
    lds_barrier();
    constexpr int PAIR_CH = D / 16;                      // 8-pair chunks per row
#pragma unroll
    for (int cc = 0; cc < PAIR_CH; cc += kThreads / 64) {
      const int c_ = cc + wave;                          // wave-uniform
      if (c_ < PAIR_CH) {
        uint64_t th[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) th[e] = p.rope_theta.t[8 * c_ + e];
#pragma unroll
        for (int k_ = 0; k_ < kRowsWG / 64; ++k_) {
          const int r_ = lane + 64 * k_;
          unsigned char* rowp = lds + r_ * QS;
          bf16x8 lo = *reinterpret_cast<const bf16x8*>(rowp + c_ * 16);
          bf16x8 hi = *reinterpret_cast<const bf16x8*>(rowp + (c_ + PAIR_CH) * 16);
          rope_rotate8(lo, hi, pos0 + qb * p.P + r_ % p.P, th);
          *reinterpret_cast<bf16x8*>(rowp + c_ * 16) = lo;
          *reinterpret_cast<bf16x8*>(rowp + (c_ + PAIR_CH) * 16) = hi;
        }
      }
    }
    lds_barrier();
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(lds + rho * QS + (ks * 16 + h * 8) * 2);
    lds_barrier();                                     // the stages may be written from here on
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m_run = -INFINITY;   // unscaled running maximum of this row
  float l_run = 0.f;         // this lane's share of the normalizer
  // S^T of the current tile, four 32-key blocks.  After the vector phase the first
  // eight values of block kb hold P^T of chunks 2 kb and 2 kb + 1 as packed bf16.
  f32x16 sacc[4];

  // ---- staging: K and V tiles straight from memory into their stages, all requested
  // by the trailing group.  Tile t of the (b, g) slice goes to stage t & 1; 1 KiB block j
  // of a stage is written by trailing wave j % 4.  *_off[i] is this lane's byte offset
  // within a tile for block gw + 4 i.  Keys at or past kv_end read as zeros (the
  // descriptors' range ends there); a lane whose 16 bytes are row padding reads at
  // 2^31, past any range the API admits (a head's slice is below 2^31 bytes), so it
  // touches no memory and writes zeros into padding no product reads.
  const size_t kv_base = (size_t)(b * p.h_kv + g) * p.T_cap * D;
  const uint32_t slice_bytes = (uint32_t)kv_end * D * 2;
  const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(p.k + kv_base, slice_bytes);
  const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(p.v + kv_base, slice_bytes);
  uint32_t k_off[L::MAXB], v_off[L::MAXB];
#pragma unroll
  for (int i = 0; i < L::MAXB; ++i) {
    const int a = (gw + 4 * i) * 1024 + lane * 16;
    const int rk = a / L::KS, ok = a - rk * L::KS;
    const int rv = a / L::VS, ov = a - rv * L::VS;
    k_off[i] = ok < D * 2 ? (uint32_t)(rk * D * 2 + ok) : 0x80000000u;
    v_off[i] = ov < D * 2 ? (uint32_t)(rv * D * 2 + ov) : 0x80000000u;
  }
  // Block i of this wave's share of tile t of K (or V) into `stage`.
  auto load_k_block = [&](unsigned char* stage, const int t, const int i) {
    if (gw + 4 * i < L::K_BLOCKS)
      load_lds16(k_rs, stage + (gw + 4 * i) * 1024, k_off[i], (uint32_t)t * kTile * D * 2);
  };
  auto load_v_block = [&](unsigned char* stage, const int t, const int i) {
    if (gw + 4 * i < L::V_BLOCKS)
      load_lds16(v_rs, stage + (gw + 4 * i) * 1024, v_off[i], (uint32_t)t * kTile * D * 2);
  };
  auto load_k_tile = [&](unsigned char* stage, const int t) {
#pragma unroll
    for (int i = 0; i < L::MAXB; ++i) load_k_block(stage, t, i);
  };
  auto load_v_tile = [&](unsigned char* stage, const int t) {
#pragma unroll
    for (int i = 0; i < L::MAXB; ++i) load_v_block(stage, t, i);
  };
  auto k_stage = [&](const int t) { return lds + (t & 1) * L::K_STAGE; };
  auto v_stage = [&](const int t) { return lds + L::V_OFF + (t & 1) * L::V_STAGE; };

  // ---- matrix phase: O^T += V^T P^T for the previous tile (PV, V stage vs_) and
  // S^T = K Q^T for this one (QK, K stage ks_), in PhaseOrder.  Operand reads run kWin
  // products ahead of the products that consume them, in an order pinned by
  // scheduling barriers.  The stages read here are never the ones the trailing
  // group's loads in flight are writing (see the pipeline below).
  constexpr int kWin = 8;
  bf16x8 ops[kWin];
  auto matrix_phase = [&](auto qk_tag, auto pv_tag, const unsigned char* __restrict__ ks_,
                          const unsigned char* __restrict__ vs_) {
    constexpr bool QK = decltype(qk_tag)::value;
    constexpr bool PV = decltype(pv_tag)::value;
    using O = PhaseOrder<D, QK, PV>;
    constexpr int N = O::N;
    auto read = [&](int j) -> bf16x8 {
      const int c = O::at(j);
      const int x = (c >> 4) & 15, y = c & 15;
      if (c >= 256) return load_vt_operand(vs_, L::VS, x, y * 32, lane);
      return *reinterpret_cast<const bf16x8*>(ks_ + (x * 32 + col) * L::KS + (y * 16 + h * 8) * 2);
    };
#pragma unroll
    for (int j = 0; j < kWin && j < N; ++j) ops[j] = read(j);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      const int c = O::at(j);
      const int x = (c >> 4) & 15, y = c & 15;
      if (c >= 256) {
        const f32x16& sp = sacc[x >> 1];
        const int e0 = 4 * (x & 1);
        typedef float f32x4_ __attribute__((ext_vector_type(4)));
        const f32x4_ w = {sp[e0], sp[e0 + 1], sp[e0 + 2], sp[e0 + 3]};
        oacc[y] = mfma32(ops[j % kWin], __builtin_bit_cast(bf16x8, w), oacc[y]);
      } else {
        sacc[x] = mfma32(ops[j % kWin], qf[y], y == 0 ? f32x16{} : sacc[x]);
      }
      if (j + kWin < N) ops[j % kWin] = read(j + kWin);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- vector phase t: online-softmax update from S^T of tile t; P^T packed in place.
  // The trailing group also requests K tile t + 2 and V tile t + 1 (the leading group
  // is then in its matrix phase t + 1).
  auto vector_phase = [&](const int t) {
    // Trailing wave gw requests its blocks of both tiles at point gw of the phase (the
    // start, after the maximum, after the first and the second block of exponentials),
    // so that one wave's loads at a time queue in the memory pipeline: a wave's later
    // instructions wait until its own loads are taken, and the other three compute.
    auto loads_at = [&](const int point) {
      if (grp == 1 && gw == point) {
        if (t + 2 < n_tiles) load_k_tile(k_stage(t + 2), t + 2);
        if (t + 1 < n_tiles) load_v_tile(v_stage(t + 1), t + 1);
      }
    };
    loads_at(0);
    const int k0 = t * kTile;
    // mask only where some key of the tile may be invisible to some row
    const bool need_mask = (p.causal && k0 + kTile - 1 > min_pos) || (k0 + kTile > len_b);
    if (need_mask) {
      // key k0 + kb * 32 + 8 (e / 4) + 4 h + e % 4 is visible iff it lies below
      // min(len_b, pos + 1) (causal) or len_b; lim moves k0 + 4 h to that side, so each
      // element takes one compare against a constant and one select
      const int lim = (p.causal ? min(len_b, pos + 1) : len_b) - k0 - 4 * h;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          sacc[kb][e] = (kb * 32 + 8 * (e >> 2) + (e & 3)) < lim ? sacc[kb][e] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
    mx = pair_max(mx);
    asm volatile("" : "+v"(mx));
    loads_at(1);
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
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = fast_exp2(fmaf(sacc[kb][e], p.c, -mc));
        sacc[kb][e] = pe;
        psum += pe;
      }
      f32x16& sv = sacc[kb];
      const bf16x8 c0 = pack_bf16x8(sv[0], sv[1], sv[2], sv[3], sv[4], sv[5], sv[6], sv[7]);
      const bf16x8 c1 = pack_bf16x8(sv[8], sv[9], sv[10], sv[11], sv[12], sv[13], sv[14], sv[15]);
      typedef float f32x4_ __attribute__((ext_vector_type(4)));
      f32x4_ w0 = __builtin_bit_cast(f32x4_, c0), w1 = __builtin_bit_cast(f32x4_, c1);
      if (kb < 2) {
        // block kb's exponentials come before the loads of point kb + 2 (the empty asm
        // keeps the compiler from moving them past the loads)
        asm volatile("" : "+v"(w0), "+v"(w1), "+v"(psum));
        loads_at(kb + 2);
      }
      sv[0] = w0[0]; sv[1] = w0[1]; sv[2] = w0[2]; sv[3] = w0[3];
      sv[4] = w1[0]; sv[5] = w1[1]; sv[6] = w1[2]; sv[7] = w1[3];
    }
    l_run += psum;
  };

  // ---- pipeline.  Slot 2t: leading group matrix phase t, trailing group vector phase
  // t - 1; slot 2t + 1: leading vector t, trailing matrix t; a workgroup barrier ends
  // every slot.  Matrix phase t reads K tile t and V tile t - 1.  At the start of slot
  // 2t the trailing group requests K tile t + 1, into the stage of K tile t - 1 (last
  // read in slot 2t - 1), and V tile t, into the stage of V tile t - 2 (last read in
  // slot 2t - 1); its matrix phase t in slot 2t + 1 reads neither of those stages, and
  // it waits for the loads at the end of that phase, before their first reader (the
  // leading group's matrix phase t + 1).  The barrier after a matrix phase waits for
  // this wave's LDS reads; the one after a vector phase, which touches no LDS, waits
  // for nothing.
  if (n_tiles > 0) {
    const auto yes = std::integral_constant<bool, true>{};
    const auto no = std::integral_constant<bool, false>{};
    if constexpr (ROPE) load_q_rotated();
    if (grp == 1) load_k_tile(k_stage(0), 0);
    wait_lds_loads();               // K tile 0, and every wave's Q fragments
    stage_barrier();
    if (grp == 1) {
      // the trailing group starts one phase late; it requests K tile 1 and V tile 0
      if (1 < n_tiles) load_k_tile(k_stage(1), 1);
      load_v_tile(v_stage(0), 0);
      stage_barrier();
    }
    matrix_phase(yes, no, k_stage(0), v_stage(1));
    if (grp == 1) wait_lds_loads();
    stage_barrier();
    vector_phase(0);
    vector_barrier();
    for (int t = 1; t < n_tiles; ++t) {
      matrix_phase(yes, yes, k_stage(t), v_stage(t - 1));
      if (grp == 1) wait_lds_loads();   // K tile t + 1, V tile t
      stage_barrier();
      vector_phase(t);
      vector_barrier();
    }
    matrix_phase(no, yes, k_stage(n_tiles), v_stage(n_tiles - 1));
    if (grp == 0) stage_barrier();  // pairs with the trailing group's last barrier
  }

  // ---- epilogue: o = u / l
  const float l_tot = pair_sum(l_run);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (row_valid && p.lse && h == 0) {
    // l_tot sums exp(scale (s - m)) with m the unscaled running maximum
    constexpr float kLn2 = 0.6931471805599453f;
    p.lse[(size_t)(b * p.h_q + head) * p.S_q + qi] =
        l_tot > 0.f ? fmaf(__builtin_amdgcn_logf(l_tot), kLn2, m_run * p.scale) : -INFINITY;
  }
  // O leaves through LDS, so that a store instruction writes whole 128-byte lines of
  // a few rows rather than 16-byte pieces of 32 rows, and with the non-temporal hint,
  // so that the output does not sit dirty in L2 when the kernel ends.  The leading
  // group uses the K stages (free after its last barrier), the trailing group the V
  // stage its last phase does not read; each wave owns 32 rows of D + 16 bytes and
  // passes its rows through in ESZ parts of D bytes.
  {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    constexpr int ESZ = OUT_BF16 ? 2 : 4;      // bytes per output value
    constexpr int RS = D + 16;                 // LDS row stride, bytes
    constexpr int DP = D / ESZ;                // d values per part
    constexpr int CPR = D / 16;                // 16-byte chunks per row part
    constexpr int RPI = 64 / CPR;              // rows per store instruction
    static_assert(4 * 32 * RS <= 2 * L::K_STAGE, "leading rows fit the K stages");
    static_assert(4 * 32 * RS <= L::V_STAGE, "trailing rows fit one V stage");
    unsigned char* const wl = lds + (grp == 0 ? 0 : L::V_OFF + (n_tiles & 1) * L::V_STAGE) + (wave & 3) * 32 * RS;
#pragma unroll
    for (int ps = 0; ps < ESZ; ++ps) {
#pragma unroll
      for (int u = ps * DP / 8; u < (ps + 1) * DP / 8; ++u) {
        // unit u: d = 8 u + 4 h + e, held in oacc[u / 4][4 (u % 4) + e]
        const int db = u / 4, j = u % 4;
        const int off = (8 * u + 4 * h - ps * DP) * ESZ;
        const float o0 = oacc[db][4 * j] * inv, o1 = oacc[db][4 * j + 1] * inv;
        const float o2 = oacc[db][4 * j + 2] * inv, o3 = oacc[db][4 * j + 3] * inv;
        if constexpr (OUT_BF16) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 w;
          w[0] = (__bf16)o0; w[1] = (__bf16)o1; w[2] = (__bf16)o2; w[3] = (__bf16)o3;
          *reinterpret_cast<bf16x4*>(wl + col * RS + off) = w;
        } else {
          *reinterpret_cast<float4*>(wl + col * RS + off) = make_float4(o0, o1, o2, o3);
        }
      }
      // the wave reads back what its own lanes wrote: order within the wave suffices
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
      for (int it = 0; it < 32 / RPI; ++it) {
        const int rw = it * RPI + lane / CPR;   // row within the wave
        const int c = lane % CPR;
        const u32x4 x = *reinterpret_cast<const u32x4*>(wl + rw * RS + c * 16);
        const int rho_ = wave * 32 + rw;
        const int qi_ = qb * p.P + rho_ % p.P;
        if (qi_ < p.S_q) {
          const int head_ = g * p.r + hc * p.hp + rho_ / p.P;
          unsigned char* orow = static_cast<unsigned char*>(p.o) + ((size_t)(b * p.h_q + head_) * p.S_q + qi_) * D * ESZ;
          __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(orow + ps * D + c * 16));
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    }
  }
}

template <int D, bool OUT_BF16, bool ROPE>
hipError_t launch_v(const PrefillParams& prm, int total, hipStream_t s) {
  constexpr int smem = PrefillLds<D>::TOTAL;
  static std::atomic<unsigned long long> lds_allowed{0};
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(prefill_bf16_kernel<D, OUT_BF16, ROPE>),
                                         smem, lds_allowed);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, OUT_BF16, ROPE>), dim3(total), dim3(kThreads), smem, s, prm);
  return hipGetLastError();
}

template <int D, bool OUT_BF16>
hipError_t launch_t(const PrefillParams& prm, int total, hipStream_t s) {
  return prm.rope ? launch_v<D, OUT_BF16, true>(prm, total, s) : launch_v<D, OUT_BF16, false>(prm, total, s);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
  PrefillParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = a.o;
  p.lse = a.lse;
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
  p.scale = a.scale;
  p.rope = a.rope_base > 0.f ? 1 : 0;
  p.rope_theta = p.rope ? make_rope_theta(a.D, a.rope_base) : RopeTheta{};
  const long long total = (long long)a.B * a.h_kv * p.n_hchunks * p.n_qblocks;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  p.xcd_remap = (total % 8 == 0) ? 1 : 0;
  if (a.D == 128) return a.out_bf16 ? launch_t<128, true>(p, (int)total, s) : launch_t<128, false>(p, (int)total, s);
  return a.out_bf16 ? launch_t<64, true>(p, (int)total, s) : launch_t<64, false>(p, (int)total, s);
}

}  // namespace gqa
