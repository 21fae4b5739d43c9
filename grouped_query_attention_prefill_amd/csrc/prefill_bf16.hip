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
// maximum, exponentials, row sums, P packed to bf16).  The 8 waves form two
// groups of four, one wave of each on every SIMD, and the second group runs one
// phase behind the first: while one wave of a SIMD keeps the matrix core busy,
// the other does its exponentials, and a workgroup barrier between phases keeps
// the two groups in step.  The groups also split the staging: the leading group
// streams K tiles and the trailing group V tiles, each through registers into
// a double-buffered LDS stage, written in the middle of the group's matrix phase
// (global loads are requested two phases before their data is written).  A
// matrix phase opens with a few QK products whose K operands were read before
// its barrier.  The ROPE instances rotate the workgroup's Q rows at their
// positions (in LDS, once the first tile's loads are issued) before the loop.
// O is written through LDS as whole 128-byte lines with the non-temporal hint.
//
// Layouts in LDS, both filled by 16-byte buffer loads that return zeros past the
// last visible key (no per-load branches):
//   K [64 keys][d_h] row-major, rows padded by 16 bytes: 16-byte operand reads
//     are conflict-free at this stride (at 32 bytes of padding they take twice
//     the cycles)
//   V [64 keys][d_h] row-major, rows padded by 32 bytes, read with transposing
//     reads that hand the PV product its V^T operand directly (those cost the
//     same at every stride and layout measured).
#include <type_traits>

#include "internal.h"
#include "mfma_common.h"
#include "rope_common.h"

namespace gqa {
namespace {

constexpr int kThreads = 512;   // 8 waves: two groups of 4, one wave of each per SIMD
constexpr int kGroup = 256;     // threads per group
constexpr int kRowsWG = 256;    // query rows per workgroup (32 per wave)
constexpr int kTile = 64;       // keys per tile

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

template <int D>
struct PrefillLds {
  static constexpr int KS = D * 2 + 16;          // K row stride, bytes
  static constexpr int VS = D * 2 + 32;          // V row stride, bytes
  static constexpr int K_STAGE = kTile * KS;
  static constexpr int V_STAGE = kTile * VS;
  static constexpr int V_OFF = 2 * K_STAGE;      // two K stages, then two V stages
  static constexpr int TOTAL = 2 * K_STAGE + 2 * V_STAGE;
};

template <int D, bool OUT_BF16, bool ROPE>
__global__ void __launch_bounds__(kThreads, 1)
prefill_bf16_kernel(PrefillParams p) {
  using L = PrefillLds<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;     // 0: leads, streams K; 1: one phase behind, streams V
  const int gtid = tid & (kGroup - 1);
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
  // rows staged in LDS (free until the first tile is stored): wave w turns the pairs
  // 8 w .. 8 w + 7 of rows lane + 64 k, so its angles are wave-uniform; then every
  // lane reads its fragments as above.  Called once the first tile's loads are in
  // flight, so their latency covers this work.
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
  f32x16 sacc[2];            // S^T of the current tile, two 32-key halves
  bf16x8 pf[4];              // P^T of the previous tile, four 16-key chunks

  // ---- staging: this group's tensor (K or V), global -> registers -> LDS
  const size_t kv_base = (size_t)(b * p.h_kv + g) * p.T_cap * D;
  const uint32_t slice_bytes = (uint32_t)kv_end * D * 2;     // keys >= kv_end read as zeros
  const __amdgpu_buffer_rsrc_t srs = make_rsrc((grp == 0 ? p.k : p.v) + kv_base, slice_bytes);
  const int s_stride = grp == 0 ? L::KS : L::VS;
  unsigned char* const s_base = lds + (grp == 0 ? 0 : L::V_OFF);
  const int s_stage = grp == 0 ? L::K_STAGE : L::V_STAGE;
  constexpr int UNITS = kTile * D / 8 / kGroup;             // 16-byte chunks per thread
  uint4 sreg[UNITS];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < UNITS; ++i) {
      const int u = gtid + kGroup * i;
      const int row = u / (D / 8), c8 = u % (D / 8);
      sreg[i] = load16(srs, (uint32_t)((t * kTile + row) * D + c8 * 8) * 2);
    }
  };
  auto store_tile = [&](int t) {
    unsigned char* dst = s_base + (t & 1) * s_stage;
#pragma unroll
    for (int i = 0; i < UNITS; ++i) {
      const int u = gtid + kGroup * i;
      const int row = u / (D / 8), c8 = u % (D / 8);
      *reinterpret_cast<uint4*>(dst + row * s_stride + c8 * 16) = sreg[i];
    }
  };

  // ---- staging duty of matrix phase t.  Leading group: K tile t + 1 to LDS, K tile
  // t + 2 requested.  Trailing group: V tile t to LDS, V tile t + 1 requested.
  // Each write goes to the stage whose previous tile both groups have finished.
  auto stage_duty = [&](const int t) {
    const int ts = grp == 0 ? t + 1 : t;
    if (ts < n_tiles) {
      store_tile(ts);
      if (ts + 1 < n_tiles) load_tile(ts + 1);
    }
  };

  // ---- matrix phase t: O^T += V^T P^T for tile t - 1 (PV) and S^T = K Q^T for tile t
  // (QK).  Operand reads run kWin ahead of the products that consume them, in an
  // order pinned by scheduling barriers, alternating QK and PV products so that no
  // accumulator is needed again before the product writing it has finished.
  constexpr int NOP = D / 8;     // operands per product kind and tile
  constexpr int kWin = 8;
  constexpr int kStageAt = 8;    // staging duty is issued after this many products
  // The first NPRE QK operands of matrix phase t are read at the end of the vector
  // phase before it, ahead of the barrier, so the phase opens with products whose
  // operands are already in registers while its V reads are still in flight.  K
  // tile t was written during the leading group's matrix phase t - 1 and a barrier
  // has passed since; its stage is next written with K tile t + 2, in matrix phase
  // t + 1 of the leading group, after both groups' matrix phase t.
  constexpr int NPRE = 4;
  bf16x8 ops[kWin];
  auto pre_read = [&](const int t) {
    const unsigned char* ks_ = lds + (t & 1) * L::K_STAGE;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NPRE; ++i)
      ops[i] = *reinterpret_cast<const bf16x8*>(ks_ + ((i & 1) * 32 + col) * L::KS + ((i >> 1) * 16 + h * 8) * 2);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto matrix_phase = [&](const int t, auto qk_tag, auto pv_tag, auto pre_tag) {
    constexpr bool QK = decltype(qk_tag)::value;
    constexpr bool PV = decltype(pv_tag)::value;
    constexpr bool PRE = decltype(pre_tag)::value;
    constexpr int N = (QK ? NOP : 0) + (PV ? NOP : 0);
    const unsigned char* ks_ = lds + (t & 1) * L::K_STAGE;
    const unsigned char* vs_ = lds + L::V_OFF + ((t - 1) & 1) * L::V_STAGE;
    // order: NPRE QK products first (their operands were read before the barrier),
    // then PV and QK alternating, then the remaining PV products
    auto is_pv = [&](int j) -> bool {
      if (!(QK && PV)) return PV;
      if (j < NPRE) return false;
      const int m = j - NPRE;
      if (m < 2 * (NOP - NPRE)) return (m & 1) == 0;
      return true;
    };
    auto idx = [&](int j) -> int {
      if (!(QK && PV)) return j;
      if (j < NPRE) return j;
      const int m = j - NPRE;
      if (m < 2 * (NOP - NPRE)) return (m & 1) == 0 ? m / 2 : NPRE + m / 2;
      return (NOP - NPRE) + (m - 2 * (NOP - NPRE));
    };
    auto read = [&](int j) -> bf16x8 {
      const int i = idx(j);
      if (is_pv(j)) return load_vt_operand(vs_, L::VS, i / (D / 32), (i % (D / 32)) * 32, lane);
      return *reinterpret_cast<const bf16x8*>(ks_ + ((i & 1) * 32 + col) * L::KS + ((i >> 1) * 16 + h * 8) * 2);
    };
#pragma unroll
    for (int j = PRE ? NPRE : 0; j < kWin && j < N; ++j) ops[j] = read(j);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      const int i = idx(j);
      if (is_pv(j)) {
        const int kc = i / (D / 32), db = i % (D / 32);
        oacc[db] = mfma32(ops[j % kWin], pf[kc], oacc[db]);
      } else {
        const int kb = i & 1, kd = i >> 1;
        sacc[kb] = mfma32(ops[j % kWin], qf[kd], kd == 0 ? f32x16{} : sacc[kb]);
      }
      if (j + kWin < N) ops[j % kWin] = read(j + kWin);
      if (j == kStageAt - 1) {
        __builtin_amdgcn_sched_barrier(0);
        stage_duty(t);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- vector phase t: online-softmax update from S^T of tile t, P^T for the next
  // matrix phase; then this group's staging duty: tile t + 1 to LDS, tile t + 2 requested
  auto vector_phase = [&](const int t) {
    const int k0 = t * kTile;
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
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const f32x16& sv = sacc[kc >> 1];
      const int e0 = 8 * (kc & 1);
      pf[kc] = pack_bf16x8(sv[e0], sv[e0 + 1], sv[e0 + 2], sv[e0 + 3], sv[e0 + 4], sv[e0 + 5], sv[e0 + 6], sv[e0 + 7]);
    }
  };

  // ---- pipeline.  Phase k of the leading group runs beside phase k - 1 of the
  // trailing one; both issue the same number of barriers.  K tile t is read in
  // matrix phase t, V tile t in matrix phase t + 1; a stage is rewritten only
  // after both groups are past its last reader.
  if (n_tiles > 0) {
    const auto yes = std::integral_constant<bool, true>{};
    const auto no = std::integral_constant<bool, false>{};
    load_tile(0);
    if constexpr (ROPE) load_q_rotated();
    if (grp == 0) {
      store_tile(0);
      if (n_tiles > 1) load_tile(1);
    }
    lds_barrier();
    if (grp == 1) lds_barrier();   // the trailing group starts one phase late
    matrix_phase(0, yes, no, no);
    lds_barrier();
    vector_phase(0);
    if (1 < n_tiles) pre_read(1);
    lds_barrier();
    for (int t = 1; t < n_tiles; ++t) {
      matrix_phase(t, yes, yes, yes);
      lds_barrier();
      vector_phase(t);
      if (t + 1 < n_tiles) pre_read(t + 1);
      lds_barrier();
    }
    matrix_phase(n_tiles, no, yes, no);
    if (grp == 0) lds_barrier();   // pairs with the trailing group's last barrier
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
