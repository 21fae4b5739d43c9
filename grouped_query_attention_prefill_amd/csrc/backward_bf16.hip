// Gradients of bf16 grouped-query prefill attention on the gfx950 matrix cores:
// dQ, dK, dV in fp32 from Q, K, V, the forward output O, its gradient dO and the
// row log-sum-exp L the forward saved.
//
// Method ([EffSeq] 在线 softmax: the forward keeps only per-row statistics, so
// probabilities are recomputed; [AttnVar] 3.5: tiles are recomputed instead of
// storing the T x T matrices).  With s = scale * q k and P = exp(s - L):
//     delta_i = sum_d dO_id O_id                       (one pass over O and dO)
//     dV_j    = sum_i P_ij dO_i
//     dS_ij   = P_ij (dO_i . V_j - delta_i)
//     dQ_i    = scale * sum_j dS_ij K_j
//     dK_j    = scale * sum_i dS_ij Q_i
// Every query head a of a group adds into the gradients of K/V head g(a)
// ([EffSeq] 分组查询注意力: r query heads read one K/V head).  The sums over the
// group stay inside one workgroup, so no atomics are used and results do not
// depend on scheduling.
//
// Two kernels recompute the probabilities independently:
//   dK/dV: a workgroup owns 64 keys of one (sequence, K/V head) and walks the
//     32-row query tiles of every query head in the group that can see those keys;
//     each wave's keys have their K and V rows in registers.  Per tile:
//     S = Q K^T and dP = dO V^T (rows = queries, one key per lane column), then
//     dV^T += dO^T P and dK^T += Q^T dS with P and dS straight from registers and
//     dO^T, Q^T read transposed from LDS.  Waves of different query-tile parities
//     add their partial sums at the end.  Head width 128 runs 16 keys per wave on
//     16x16x32 products, three waves per SIMD (bwd_dkdv16_kernel); head width 64
//     runs 32 keys per wave on 32x32x16 products, one wave per SIMD.
//   dQ: a workgroup owns 256 query rows (heads x positions of one group, as in
//     the forward), 32 per wave; Q and dO rows stay in registers and 64-key tiles
//     of K and V reach LDS through buffer loads that write it directly
//     (double-buffered, the next tile requested as a tile's work starts), each
//     worked in two 32-key halves (S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T).  It also forms delta for its rows (each row lives in
//     exactly one dQ workgroup) and stores it, so it runs first and the dK/dV
//     kernel reads delta from there.
#include <type_traits>

#include "internal.h"
#include "mfma_common.h"

namespace gqa {
namespace {

constexpr int kBwdThreads = 256;   // 4 waves
constexpr int kKeyBlock = 64;      // keys per dK/dV workgroup
constexpr int kQTile = 32;         // query rows per dK/dV tile
constexpr int kDqRows = 256;       // query rows per dQ workgroup
constexpr int kDqThreads = 512;    // 8 waves of 32 rows
constexpr int kDqTile = 64;        // keys per dQ tile

struct BwdParams {
  const uint16_t* q;       // (B, h_q, T, D) bf16
  const uint16_t* k;       // (B, h_kv, T, D)
  const uint16_t* v;
  const void* o;           // (B, h_q, T, D) fp32 or bf16
  const uint16_t* d_o;     // (B, h_q, T, D) bf16
  const float* lse;        // (B, h_q, T)
  float* delta;            // (B, h_q, T) workspace
  float* dq;               // (B, h_q, T, D) fp32
  float* dk;               // (B, h_kv, T, D) fp32
  float* dv;
  const int32_t* kv_lens;
  int B, h_q, h_kv, r, T, causal, o_bf16;
  int dq_delta;            // the dQ kernel forms delta from its own rows (O 16-byte aligned) and stores it
  int hp, P, n_qblocks, n_hchunks;   // dQ row packing (as the forward)
  float scale, c;                    // c = scale * log2(e)
};

__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// dK/dV work item -> (query head, query tile).  Wave-uniform, which the buffer
// descriptors built from it must be (readfirstlane states it to the compiler).
__device__ __forceinline__ void dkdv_item(int it, int g, int r, int per_head, int qt0, int& head, int& qt) {
  head = __builtin_amdgcn_readfirstlane(g * r + it / per_head);
  qt = __builtin_amdgcn_readfirstlane(qt0 + it % per_head);
}

// ---------------------------------------------------------------------------
// delta_i = sum_d dO_id O_id, one wave per row with element loads: the pass for an O
// that is not 16-byte aligned (otherwise the dQ kernel forms delta from its rows)
template <int D>
__global__ void __launch_bounds__(256)
bwd_delta_kernel(BwdParams p) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const long long n_rows = (long long)p.B * p.h_q * p.T;
  if (row >= n_rows) return;
  float acc = 0.f;
  for (int d = lane; d < D; d += 64) {
    const float o = p.o_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p.o)[row * D + d])
                             : static_cast<const float*>(p.o)[row * D + d];
    acc = fmaf(bf16_to_f32(p.d_o[row * D + d]), o, acc);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) p.delta[row] = acc;
}

// ---------------------------------------------------------------------------
template <int D>
struct DkdvLds {
  static constexpr int TS = D * 2 + 32;            // tile row stride, bytes
  static constexpr int TILE = kQTile * TS;
  static constexpr int REGION = 2 * TILE + 2 * kQTile * 4;   // Q tile, dO tile, L, delta
  static constexpr int STAGING = 2 * 2 * REGION;             // two parities x two stages
  static constexpr int REDUCE = 2 * 2 * (D / 32) * 16 * 64 * 4;   // two waves x (dK, dV) accumulators
  static constexpr int TOTAL = STAGING > REDUCE ? STAGING : REDUCE;
};

template <int D>
__global__ void __launch_bounds__(kBwdThreads, 1)
bwd_dkdv_kernel(BwdParams p) {
  using L = DkdvLds<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave & 1;          // key half of the block
  const int qw = wave >> 1;         // query-tile parity
  const int h = lane >> 5, col = lane & 31;
  const int gtid = tid & 127;       // thread index within the parity pair
  // parameters the lambdas below use, as scalars (a reference to the whole
  // parameter block would force it into private memory)
  const int T = p.T, h_q = p.h_q, r = p.r, causal = p.causal;
  const float c2 = p.c;
  const uint16_t* const qp = p.q;
  const uint16_t* const dop = p.d_o;
  const float* const lsep = p.lse;
  const float* const deltap = p.delta;

  // heaviest key blocks first: under a causal mask the first keys are seen by every row
  const int n_bg = p.B * p.h_kv;
  const int kb = blockIdx.x / n_bg;
  const int bg = blockIdx.x % n_bg;
  const int g = bg % p.h_kv, b = bg / p.h_kv;
  const int len_b = clampi(p.kv_lens ? p.kv_lens[b] : p.T, 0, p.T);
  const int key0 = kb * kKeyBlock + kw * 32;        // first key of this wave
  const int key = key0 + col;                       // this lane's key

  // K and V rows of this wave's keys: B operands of S = Q K^T and dP = dO V^T
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const size_t base = ((size_t)(b * p.h_kv + g) * p.T + key) * D;
    const bool ok = key < len_b;
#pragma unroll
    for (int kd = 0; kd < D / 16; ++kd) {
      uint4 x = make_uint4(0, 0, 0, 0), y = make_uint4(0, 0, 0, 0);
      if (ok) {
        x = *reinterpret_cast<const uint4*>(p.k + base + kd * 16 + h * 8);
        y = *reinterpret_cast<const uint4*>(p.v + base + kd * 16 + h * 8);
      }
      kf[kd] = __builtin_bit_cast(bf16x8, x);
      vf[kd] = __builtin_bit_cast(bf16x8, y);
    }
  }
  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) { dkacc[db][e] = 0.f; dvacc[db][e] = 0.f; }

  // query tiles that can see some key of the block: every head of the group, rows
  // from the block's first key on (causal) or all rows
  const int n_qt = (p.T + kQTile - 1) / kQTile;
  const int qt0 = (p.causal && kb * kKeyBlock < len_b) ? (kb * kKeyBlock) / kQTile : 0;
  const int per_head = n_qt - qt0;
  const int n_items = (kb * kKeyBlock < len_b) ? p.r * per_head : 0;
  const int n_steps = (n_items + 1) / 2;

  // staging of one item (head, query tile) into region (qw, stage) by the two waves of parity qw
  constexpr int UNITS = kQTile * D / 8 / 128;        // 16-byte chunks per thread per tensor
  // two register sets: an item's global loads are issued two steps before its
  // data goes to LDS, so HBM latency hides behind two steps of products
  uint4 qreg[2][UNITS], oreg[2][UNITS];
  float lreg[2] = {0.f, 0.f}, dreg[2] = {0.f, 0.f};
  auto load_item = [&](int it, auto set_tag) __attribute__((always_inline)) {
    constexpr int set = decltype(set_tag)::value;
    // past the last item the loads still issue, through empty descriptors that
    // return zeros: every step then issues the same loads, which lets the compiler
    // count exactly which of them a later wait needs
    const bool valid = it < n_items;
    int head, qt;
    dkdv_item(valid ? it : 0, g, r, per_head, qt0, head, qt);
    const size_t rbase = ((size_t)(b * h_q + head) * T) * D;
    const uint32_t bytes = valid ? (uint32_t)T * D * 2 : 0u;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qp + rbase, bytes);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(dop + rbase, bytes);
#pragma unroll
    for (int i = 0; i < UNITS; ++i) {
      const int u = gtid + 128 * i;
      const int row = u / (D / 8), c8 = u % (D / 8);
      const uint32_t off = (uint32_t)(((qt * kQTile + row) * D + c8 * 8) * 2);
      qreg[set][i] = load16(qr, off);
      oreg[set][i] = load16(dr, off);
    }
    const int qi = qt * kQTile + (gtid & 31);
    const size_t li = (size_t)(b * h_q + head) * T;
    // every thread fetches its row's two statistics (threads 0-31 store L, 32-63
    // delta); rows at or past T read 0, and the edge mask drops them
    const uint32_t sbytes = valid ? (uint32_t)T * 4 : 0u;
    lreg[set] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(lsep + li, sbytes),
                                                                             qi * 4, 0, 0));
    dreg[set] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(deltap + li, sbytes),
                                                                             qi * 4, 0, 0));
  };
  auto store_item = [&](int it, int stage, auto set_tag) __attribute__((always_inline)) {
    constexpr int set = decltype(set_tag)::value;
    if (it >= n_items) return;
    unsigned char* rg = lds + (qw * 2 + stage) * L::REGION;
#pragma unroll
    for (int i = 0; i < UNITS; ++i) {
      const int u = gtid + 128 * i;
      const int row = u / (D / 8), c8 = u % (D / 8);
      *reinterpret_cast<uint4*>(rg + row * L::TS + c8 * 16) = qreg[set][i];
      *reinterpret_cast<uint4*>(rg + L::TILE + row * L::TS + c8 * 16) = oreg[set][i];
    }
    float* lv = reinterpret_cast<float*>(rg + 2 * L::TILE);
    if (gtid < 32) lv[gtid] = lreg[set];
    else if (gtid < 64) lv[kQTile + (gtid - 32)] = dreg[set];
  };

  // one item on this wave: 32 query rows x 32 keys, 32 products
  auto compute_item = [&](int it, int stage) __attribute__((always_inline)) {
    int head, qt;
    dkdv_item(it, g, r, per_head, qt0, head, qt);
    (void)head;
    const unsigned char* rg = lds + (qw * 2 + stage) * L::REGION;
    const unsigned char* qs = rg;
    const unsigned char* os = rg + L::TILE;
    const float* lv = reinterpret_cast<const float*>(rg + 2 * L::TILE);
    f32x16 sacc, dpacc;
#pragma unroll
    for (int kd = 0; kd < D / 16; ++kd) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(qs + col * L::TS + (kd * 16 + h * 8) * 2);
      const bf16x8 o = *reinterpret_cast<const bf16x8*>(os + col * L::TS + (kd * 16 + h * 8) * 2);
      sacc = mfma32(a, kf[kd], kd == 0 ? f32x16{} : sacc);
      dpacc = mfma32(o, vf[kd], kd == 0 ? f32x16{} : dpacc);
    }
    // rows of element e: query 8 (e / 4) + 4 h + e % 4 of the tile; column: this lane's key
    const int q0 = qt * kQTile;
    const bool edge = (causal && key0 + 31 > q0) || (key0 + 32 > len_b) || (q0 + kQTile > T);
    bf16x8 pf[2], dsf[2];
    float lq[16], dl[16];                 // L and delta of the 16 rows this lane's elements sit in
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      const float4 l4 = *reinterpret_cast<const float4*>(lv + 8 * jq + 4 * h);
      const float4 d4 = *reinterpret_cast<const float4*>(lv + kQTile + 8 * jq + 4 * h);
      lq[4 * jq] = l4.x; lq[4 * jq + 1] = l4.y; lq[4 * jq + 2] = l4.z; lq[4 * jq + 3] = l4.w;
      dl[4 * jq] = d4.x; dl[4 * jq + 1] = d4.y; dl[4 * jq + 2] = d4.z; dl[4 * jq + 3] = d4.w;
    }
    // P = exp2(c s - L log2 e); masked entries take exp2(-inf) = 0.  Inside the
    // key range, below the diagonal and above T every row sees key 0, so L is
    // finite and no mask is needed off the edge tiles.
    auto probs = [&](auto masked_tag) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float arg = fmaf(sacc[e], c2, -lq[e] * kLog2e);
        if constexpr (decltype(masked_tag)::value) {
          const int qrow = q0 + 8 * (e >> 2) + 4 * h + (e & 3);
          const bool vis = (lq[e] != -INFINITY) & (key < len_b) & (qrow < T) & (!causal | (key <= qrow));
          arg = vis ? arg : -INFINITY;
        }
        const float pr = fast_exp2(arg);
        sacc[e] = pr;
        dpacc[e] = pr * (dpacc[e] - dl[e]);
      }
    };
    if (edge) probs(std::true_type{});
    else probs(std::false_type{});
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int e0 = 8 * kc;
      pf[kc] = pack_bf16x8(sacc[e0], sacc[e0 + 1], sacc[e0 + 2], sacc[e0 + 3], sacc[e0 + 4], sacc[e0 + 5],
                           sacc[e0 + 6], sacc[e0 + 7]);
      dsf[kc] = pack_bf16x8(dpacc[e0], dpacc[e0 + 1], dpacc[e0 + 2], dpacc[e0 + 3], dpacc[e0 + 4],
                            dpacc[e0 + 5], dpacc[e0 + 6], dpacc[e0 + 7]);
    }
    // dV^T += dO^T P and dK^T += Q^T dS; operands read transposed in the row order
    // the accumulator layout hands P and dS over in
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 ot = load_vt_operand(os, L::TS, kc, db * 32, lane);
        const bf16x8 qt_ = load_vt_operand(qs, L::TS, kc, db * 32, lane);
        dvacc[db] = mfma32(ot, pf[kc], dvacc[db]);
        dkacc[db] = mfma32(qt_, dsf[kc], dkacc[db]);
      }
  };

  // ---- pipeline: step s handles items 2s (parity 0) and 2s + 1 (parity 1).  At step
  // s, LDS stage s & 1 holds this parity's item of step s, register set (s + 1) & 1
  // holds the item of step s + 1 (written to the other stage after the products),
  // and register set s & 1 takes the item of step s + 2.
  const std::integral_constant<int, 0> set0{};
  const std::integral_constant<int, 1> set1{};
  load_item(qw, set0);
  load_item(2 + qw, set1);
  store_item(qw, 0, set0);
  lds_barrier();
  // The K and V fragments are in registers before the loop starts (the staging
  // above waited for them); the empty asm makes that explicit to the compiler,
  // which otherwise carries their pending loads into the loop and waits there
  // for every load in flight, prefetches included.
#pragma unroll
  for (int kd = 0; kd < D / 16; ++kd) asm volatile("" : "+v"(kf[kd]), "+v"(vf[kd]));
  // steps run in pairs (an odd count ends with an empty step) so that both
  // register sets are named at compile time
  for (int s = 0; s < n_steps; s += 2) {
    {
      const int it = 2 * s + qw;
      load_item(it + 4, set0);
      if (it < n_items) compute_item(it, 0);
      store_item(it + 2, 1, set1);
      lds_barrier();
    }
    {
      const int it = 2 * (s + 1) + qw;
      load_item(it + 4, set1);
      if (it < n_items) compute_item(it, 1);
      store_item(it + 2, 0, set0);
      lds_barrier();
    }
  }

  // ---- add the two parities' partial sums, then write dK = scale dK^T^T and dV
  float* red = reinterpret_cast<float*>(lds);      // [kw][dk | dv][db][e][lane]
  if (qw == 1) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        red[(((kw * 2 + 0) * (D / 32) + db) * 16 + e) * 64 + lane] = dkacc[db][e];
        red[(((kw * 2 + 1) * (D / 32) + db) * 16 + e) * 64 + lane] = dvacc[db][e];
      }
  }
  lds_barrier();
  if (qw == 0 && key < p.T) {
    const size_t obase = ((size_t)(b * p.h_kv + g) * p.T + key) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float kk[4], vv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * j + i;
          kk[i] = (dkacc[db][e] + red[(((kw * 2 + 0) * (D / 32) + db) * 16 + e) * 64 + lane]) * p.scale;
          vv[i] = dvacc[db][e] + red[(((kw * 2 + 1) * (D / 32) + db) * 16 + e) * 64 + lane];
        }
        const int d0 = db * 32 + 8 * j + 4 * h;
        *reinterpret_cast<float4*>(p.dk + obase + d0) = make_float4(kk[0], kk[1], kk[2], kk[3]);
        *reinterpret_cast<float4*>(p.dv + obase + d0) = make_float4(vv[0], vv[1], vv[2], vv[3]);
      }
  }
}

// ---------------------------------------------------------------------------
// dK/dV for head width 128 on 16x16x32 products, three waves per SIMD.  A
// workgroup owns 64 keys of one (sequence, K/V head); its 12 waves are 4 key
// quarters (16 keys each, K and V rows in registers) x 3 query-tile parities.  The
// Q and dO tiles of a parity's item (32 rows of one query head) reach LDS through
// buffer loads that write it directly, two items ahead (three stages per parity),
// and serve the parity's four waves.  16 keys per wave keep the dK^T and dV^T
// accumulators at 64 registers, so the kernel fits 170 registers and three waves
// share each SIMD.  Per item and wave:
//     S, dP (32 rows x 16 keys)   A: Q / dO rows from LDS, B: K / V fragments
//     dV^T, dK^T (128 d x 16 keys) += dO^T P, Q^T dS   A: transposing LDS reads,
//                                                      B: P / dS from registers
// 16x16x32 lane layouts: A (16 x 32) lane l holds A[l % 16][8 (l / 16) + t];
// B (32 x 16) lane l holds B[8 (l / 16) + t][l % 16]; C lane l, element j holds
// C[4 (l / 16) + j][l % 16].  The score block rb (rows 16 rb .. 16 rb + 15) thus
// hands lane l the rows 16 rb + 4 (l / 16) + j of its key, and slot t of the B
// operand of the second pair of products is row rowof(l / 16, t) =
// 4 (l / 16) + t (t < 4) or 16 + 4 (l / 16) + t - 4, the order in which the
// transposing reads below fetch dO^T and Q^T.
// Tile rows are 256 bytes with their 16-byte chunks permuted by chunk ^ swz(row),
// which puts the 16 rows of one chunk that a 16-byte row read takes, and the 8 rows
// x 32 bytes a half-wave of a transposing read takes, on distinct 16-byte bank
// groups of a 256-byte row of banks.
constexpr int kDk16Par = 3;        // query-tile parities (waves per SIMD)
constexpr int kDk16Threads = 256 * kDk16Par;
constexpr int kDk16Stages = 3;
constexpr int kDk16Loads = 5;      // load instructions per wave and item: 2 Q, 2 dO, 1 statistics

struct Dkdv16Lds {
  static constexpr int TILE = kQTile * 256;
  static constexpr int STATS = 4 * 256;           // L, delta, and a copy of each
  static constexpr int STAGE = 2 * TILE + STATS;
  static constexpr int TOTAL = kDk16Par * kDk16Stages * STAGE;
  static_assert(4 * 64 * 64 * 4 <= TOTAL, "the reduction of the parities fits");
};

__device__ __forceinline__ int dk16_swz(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }

typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One 16-byte-per-lane buffer load written straight into LDS: lane i's 16 bytes from
// byte voff + soff of the descriptor's range land at dst + 16 i (dst wave-uniform).
__device__ __forceinline__ void bwd_load_lds16(__amdgpu_buffer_rsrc_t r, unsigned char* dst, uint32_t voff,
                                               uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}
// 4 bytes per lane: lane i's dword lands at dst + 4 i
__device__ __forceinline__ void dk16_load_lds4(__amdgpu_buffer_rsrc_t r, unsigned char* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 4, voff, soff, 0, 0);
}

// A operand (16 d x 32 rows) of dV^T += dO^T P or dK^T += Q^T dS for d block dblk:
// two transposing reads; source lane (group G, j, q) points at row 4 G + j (then
// + 16), columns 16 dblk + 4 q .. + 3, so output lane l receives, as slots
// 0..3 and 4..7, tile[rowof(l / 16, t)][16 dblk + l % 16].
__device__ __forceinline__ bf16x8 dk16_tr_operand(const unsigned char* __restrict__ tile, int dblk, int lane) {
  const int G = lane >> 4, s = lane & 15;
  const int R = 4 * G + (s >> 2), q = s & 3;
  const int c = 2 * dblk + (q >> 1);
  const unsigned char* a = tile + R * 256 + ((c ^ dk16_swz(R)) << 4) + 8 * (q & 1);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 16 * 256));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, r);
}

__global__ void __launch_bounds__(kDk16Threads, 1)
bwd_dkdv16_kernel(BwdParams p) {
  constexpr int D = 128;
  using L = Dkdv16Lds;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kq = wave & 3;          // key quarter
  const int qw = wave >> 2;         // query-tile parity
  const int G = lane >> 4, li = lane & 15;
  const int T = p.T, h_q = p.h_q, r = p.r, causal = p.causal;
  const float c2 = p.c;
  const uint16_t* const qp = p.q;
  const uint16_t* const dop = p.d_o;
  const float* const lsep = p.lse;
  const float* const deltap = p.delta;

  const int n_bg = p.B * p.h_kv;
  const int kb = blockIdx.x / n_bg;
  const int bg = blockIdx.x % n_bg;
  const int g = bg % p.h_kv, b = bg / p.h_kv;
  const int len_b = clampi(p.kv_lens ? p.kv_lens[b] : p.T, 0, p.T);
  const int key0 = kb * kKeyBlock + kq * 16;        // first key of this wave
  const int key = key0 + li;                        // this lane's key

  bf16x8 kf[D / 32], vf[D / 32];
  {
    const size_t base = ((size_t)(b * p.h_kv + g) * p.T + key) * D;
    const bool ok = key < len_b;
#pragma unroll
    for (int kd = 0; kd < D / 32; ++kd) {
      uint4 x = make_uint4(0, 0, 0, 0), y = make_uint4(0, 0, 0, 0);
      if (ok) {
        x = *reinterpret_cast<const uint4*>(p.k + base + kd * 32 + G * 8);
        y = *reinterpret_cast<const uint4*>(p.v + base + kd * 32 + G * 8);
      }
      kf[kd] = __builtin_bit_cast(bf16x8, x);
      vf[kd] = __builtin_bit_cast(bf16x8, y);
    }
  }
  f32x4 dkacc[D / 16], dvacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) { dkacc[db][e] = 0.f; dvacc[db][e] = 0.f; }

  const int n_qt = (p.T + kQTile - 1) / kQTile;
  const int qt0 = (p.causal && kb * kKeyBlock < len_b) ? (kb * kKeyBlock) / kQTile : 0;
  const int per_head = n_qt - qt0;
  const int n_items = (kb * kKeyBlock < len_b) ? p.r * per_head : 0;
  const int n_steps = (n_items + kDk16Par - 1) / kDk16Par;

  // staging: wave kq writes 1 KiB blocks kq and kq + 4 (rows 4 j .. 4 j + 3) of the Q
  // and the dO tile; lane i of block j fills physical chunk i % 16 of row 4 j + i / 16
  uint32_t voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 4 * (kq + 4 * i) + (lane >> 4);
    voff[i] = (uint32_t)(row * 256 + (((lane & 15) ^ dk16_swz(row)) << 4));
  }
  const uint32_t svoff = lane < 32 ? (uint32_t)lane * 4 : 0x80000000u;
  const float* const stat_src = (kq & 1) ? deltap : lsep;
  auto stage_at = [&](int st) { return lds + (qw * kDk16Stages + st) * L::STAGE; };
  auto issue = [&](int it, unsigned char* __restrict__ stg) __attribute__((always_inline)) {
    const bool valid = it < n_items;
    int head, qt;
    dkdv_item(valid ? it : 0, g, r, per_head, qt0, head, qt);
    const size_t rbase = ((size_t)(b * h_q + head) * T) * D;
    const uint32_t bytes = valid ? (uint32_t)T * D * 2 : 0u;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qp + rbase, bytes);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(dop + rbase, bytes);
    const uint32_t soff = (uint32_t)qt * kQTile * D * 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      bwd_load_lds16(qr, stg + (kq + 4 * i) * 1024, voff[i], soff);
      bwd_load_lds16(dr, stg + L::TILE + (kq + 4 * i) * 1024, voff[i], soff);
    }
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(stat_src + (size_t)(b * h_q + head) * T, valid ? (uint32_t)T * 4 : 0u);
    dk16_load_lds4(sr, stg + 2 * L::TILE + kq * 256, svoff, (uint32_t)qt * kQTile * 4);
  };

  auto compute = [&](int it, const unsigned char* __restrict__ stg) __attribute__((always_inline)) {
    int head, qt;
    dkdv_item(it, g, r, per_head, qt0, head, qt);
    (void)head;
    const unsigned char* qs = stg;
    const unsigned char* os = stg + L::TILE;
    const float* lv = reinterpret_cast<const float*>(stg + 2 * L::TILE);
    const float* dl_ = lv + 64;
    f32x4 sacc[2], dpacc[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kd = 0; kd < D / 32; ++kd) {
        const int row = 16 * rb + li;
        const int off = row * 256 + (((4 * kd + G) ^ dk16_swz(row)) << 4);
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(qs + off);
        const bf16x8 o = *reinterpret_cast<const bf16x8*>(os + off);
        sacc[rb] = mfma16(a, kf[kd], kd == 0 ? f32x4{} : sacc[rb]);
        dpacc[rb] = mfma16(o, vf[kd], kd == 0 ? f32x4{} : dpacc[rb]);
      }
    const int q0 = qt * kQTile;
    const bool edge = (causal && key0 + 15 > q0) || (key0 + 16 > len_b) || (q0 + kQTile > T);
    float lq[8], dq_[8];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float4 l4 = *reinterpret_cast<const float4*>(lv + 16 * rb + 4 * G);
      const float4 d4 = *reinterpret_cast<const float4*>(dl_ + 16 * rb + 4 * G);
      lq[4 * rb] = l4.x; lq[4 * rb + 1] = l4.y; lq[4 * rb + 2] = l4.z; lq[4 * rb + 3] = l4.w;
      dq_[4 * rb] = d4.x; dq_[4 * rb + 1] = d4.y; dq_[4 * rb + 2] = d4.z; dq_[4 * rb + 3] = d4.w;
    }
    auto probs = [&](auto masked_tag) __attribute__((always_inline)) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * rb + j;
          float arg = fmaf(sacc[rb][j], c2, -lq[e] * kLog2e);
          if constexpr (decltype(masked_tag)::value) {
            const int qrow = q0 + 16 * rb + 4 * G + j;
            const bool vis = (lq[e] != -INFINITY) & (key < len_b) & (qrow < T) & (!causal | (key <= qrow));
            arg = vis ? arg : -INFINITY;
          }
          const float pr = fast_exp2(arg);
          sacc[rb][j] = pr;
          dpacc[rb][j] = pr * (dpacc[rb][j] - dq_[e]);
        }
    };
    if (edge) probs(std::true_type{});
    else probs(std::false_type{});
    const bf16x8 pf = pack_bf16x8(sacc[0][0], sacc[0][1], sacc[0][2], sacc[0][3], sacc[1][0], sacc[1][1], sacc[1][2],
                                  sacc[1][3]);
    const bf16x8 dsf = pack_bf16x8(dpacc[0][0], dpacc[0][1], dpacc[0][2], dpacc[0][3], dpacc[1][0], dpacc[1][1],
                                   dpacc[1][2], dpacc[1][3]);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const bf16x8 ot = dk16_tr_operand(os, db, lane);
      const bf16x8 qt_ = dk16_tr_operand(qs, db, lane);
      dvacc[db] = mfma16(ot, pf, dvacc[db]);
      dkacc[db] = mfma16(qt_, dsf, dkacc[db]);
    }
  };

  auto step_barrier = []() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS reads are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // vmcnt(kDk16Loads): all but the loads of the last item issued have landed
  auto wait_but_last = []() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70 | kDk16Loads);
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- pipeline: step s computes item 2 s + qw on stage s % 3, after requesting item
  // 2 (s + 2) + qw into stage (s + 2) % 3 (last read in step s - 1, before the barrier
  // that ended it).  Every step issues the same loads (past the last item through empty
  // descriptors, which write zeros), so the wait at its end counts exactly.
  issue(qw, stage_at(0));
  issue(kDk16Par + qw, stage_at(1));
#pragma unroll
  for (int kd = 0; kd < D / 32; ++kd) asm volatile("" : "+v"(kf[kd]), "+v"(vf[kd]));
  wait_but_last();
  step_barrier();
  int st = 0;
  for (int s = 0; s < n_steps; ++s) {
    const int st2 = st >= 1 ? st - 1 : st + 2;       // (s + 2) % 3
    issue(kDk16Par * (s + 2) + qw, stage_at(st2));
    const int it = kDk16Par * s + qw;
    if (it < n_items) compute(it, stage_at(st));
    wait_but_last();
    step_barrier();
    st = st == 2 ? 0 : st + 1;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);               // no load into LDS is left in flight
  step_barrier();

  // ---- add the parities' partial sums (parities 1 .. kDk16Par - 1 one after another
  // into parity 0's registers), then write dK = scale dK^T^T and dV
  float* red = reinterpret_cast<float*>(lds);       // [kq][dk | dv][db][j][lane]
  for (int src = 1; src < kDk16Par; ++src) {
    if (qw == src) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          red[(((kq * 2 + 0) * (D / 16) + db) * 4 + j) * 64 + lane] = dkacc[db][j];
          red[(((kq * 2 + 1) * (D / 16) + db) * 4 + j) * 64 + lane] = dvacc[db][j];
        }
    }
    lds_barrier();
    if (qw == 0) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dkacc[db][j] += red[(((kq * 2 + 0) * (D / 16) + db) * 4 + j) * 64 + lane];
          dvacc[db][j] += red[(((kq * 2 + 1) * (D / 16) + db) * 4 + j) * 64 + lane];
        }
    }
    lds_barrier();
  }
  if (qw == 0 && key < p.T) {
    const size_t obase = ((size_t)(b * p.h_kv + g) * p.T + key) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      float kk[4], vv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kk[j] = dkacc[db][j] * p.scale;
        vv[j] = dvacc[db][j];
      }
      const int d0 = db * 16 + 4 * G;
      *reinterpret_cast<float4*>(p.dk + obase + d0) = make_float4(kk[0], kk[1], kk[2], kk[3]);
      *reinterpret_cast<float4*>(p.dv + obase + d0) = make_float4(vv[0], vv[1], vv[2], vv[3]);
    }
  }
}

// ---------------------------------------------------------------------------
template <int D>
struct DqLds {
  static constexpr int KTS = D * 2 + 32;           // K tile: read as rows and transposed
  static constexpr int VTS = D * 2 + 16;           // V tile: read as rows
  static constexpr int K_BYTES = kDqTile * KTS;
  static constexpr int STAGE = K_BYTES + kDqTile * VTS;
  static constexpr int TOTAL = 2 * STAGE;
  static constexpr int K_BLOCKS = K_BYTES / 1024;                  // 1 KiB load blocks per stage
  static constexpr int V_BLOCKS = kDqTile * VTS / 1024;
  static constexpr int MAXB = (K_BLOCKS + 7) / 8;                  // blocks per wave and tensor
  static_assert(K_BYTES % 1024 == 0 && (kDqTile * VTS) % 1024 == 0, "stages are whole 1 KiB blocks");
  static_assert(K_BLOCKS >= V_BLOCKS, "the K part is the larger");
};

template <int D>
__global__ void __launch_bounds__(kDqThreads, 1)
bwd_dq_kernel(BwdParams p) {
  using L = DqLds<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;

  // heaviest query blocks first across every (sequence, K/V head, head chunk): the
  // dispatcher starts workgroups in grid order, so the long rows of all heads spread
  // over the chip first and short ones fill in behind them
  const int n_bgh = p.B * p.h_kv * p.n_hchunks;
  const int qb = p.n_qblocks - 1 - (int)(blockIdx.x / n_bgh);
  const int bgh = blockIdx.x % n_bgh;
  const int hc = bgh % p.n_hchunks;
  const int bg = bgh / p.n_hchunks;
  const int g = bg % p.h_kv, b = bg / p.h_kv;
  const int len_b = clampi(p.kv_lens ? p.kv_lens[b] : p.T, 0, p.T);

  const int rho = wave * 32 + col;
  const int head = g * p.r + hc * p.hp + rho / p.P;
  const int qi = qb * p.P + rho % p.P;
  const bool row_valid = qi < p.T;
  const size_t rrow = (size_t)(b * p.h_q + head) * p.T + qi;

  bf16x8 qf[D / 16], of[D / 16];
#pragma unroll
  for (int kd = 0; kd < D / 16; ++kd) {
    uint4 x = make_uint4(0, 0, 0, 0), y = make_uint4(0, 0, 0, 0);
    if (row_valid) {
      x = *reinterpret_cast<const uint4*>(p.q + rrow * D + kd * 16 + h * 8);
      y = *reinterpret_cast<const uint4*>(p.d_o + rrow * D + kd * 16 + h * 8);
    }
    qf[kd] = __builtin_bit_cast(bf16x8, x);
    of[kd] = __builtin_bit_cast(bf16x8, y);
  }
  const float lrow = row_valid ? p.lse[rrow] : -INFINITY;
  float drow = 0.f;
  if (p.dq_delta) {
    // delta = sum_d dO O for this row: each lane of the pair holds the d values
    // 16 kd + 8 h .. + 7 of dO in of[kd]; O's matching 8 values come from memory
    if (row_valid) {
#pragma unroll
      for (int kd = 0; kd < D / 16; ++kd) {
        float o8[8];
        const size_t e0 = rrow * D + kd * 16 + h * 8;
        if (p.o_bf16) {
          const uint4 ov = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.o) + e0);
          const uint32_t w[4] = {ov.x, ov.y, ov.z, ov.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) { o8[2 * j] = __uint_as_float(w[j] << 16); o8[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u); }
        } else {
          const float4 a = reinterpret_cast<const float4*>(static_cast<const float*>(p.o) + e0)[0];
          const float4 c = reinterpret_cast<const float4*>(static_cast<const float*>(p.o) + e0)[1];
          o8[0] = a.x; o8[1] = a.y; o8[2] = a.z; o8[3] = a.w; o8[4] = c.x; o8[5] = c.y; o8[6] = c.z; o8[7] = c.w;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) drow = fmaf((float)of[kd][j], o8[j], drow);
      }
    }
    drow = pair_sum(drow);
    if (row_valid && h == 0) p.delta[rrow] = drow;
  } else if (row_valid) {
    drow = p.delta[rrow];
  }
  // a row outside the sequence, or one that sees no key, has L = -inf; its exp2
  // arguments are then made -inf so that all of its P are 0
  const float lc = lrow != -INFINITY ? lrow * kLog2e : INFINITY;
  const int causal = p.causal;
  const float c2 = p.c;

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dqacc[db][e] = 0.f;

  const int first_q = qb * p.P;
  const int last_q = min(first_q + p.P, p.T) - 1;
  const int kv_end = p.causal ? min(len_b, last_q + 1) : len_b;
  const int n_tiles = (kv_end + kDqTile - 1) / kDqTile;

  const size_t kv_base = (size_t)(b * p.h_kv + g) * p.T * D;
  const uint32_t slice = (uint32_t)kv_end * D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + kv_base, slice);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + kv_base, slice);
  // ---- staging: K and V tiles straight from memory into their stages with buffer
  // loads that write LDS directly.  1 KiB block j of a stage's K (V) part is written by
  // wave j % 8; *_off[i] is this lane's byte offset within a tile for block wave + 8 i.
  // Keys at or past kv_end read as zeros (the descriptors' range ends there); a lane
  // whose 16 bytes are row padding reads at 2^31, outside any range the API admits, so
  // it touches no memory and writes zeros into padding no product reads.
  uint32_t k_off[L::MAXB], v_off[L::MAXB];
#pragma unroll
  for (int i = 0; i < L::MAXB; ++i) {
    const int a = (wave + 8 * i) * 1024 + lane * 16;
    const int rk = a / L::KTS, ok = a - rk * L::KTS;
    const int rv = a / L::VTS, ov = a - rv * L::VTS;
    k_off[i] = ok < D * 2 ? (uint32_t)(rk * D * 2 + ok) : 0x80000000u;
    v_off[i] = ov < D * 2 ? (uint32_t)(rv * D * 2 + ov) : 0x80000000u;
  }
  auto load_tile = [&](unsigned char* __restrict__ stage, int t) __attribute__((always_inline)) {
    const uint32_t soff = (uint32_t)t * kDqTile * D * 2;
#pragma unroll
    for (int i = 0; i < L::MAXB; ++i) {
      if (wave + 8 * i < L::K_BLOCKS) bwd_load_lds16(krs, stage + (wave + 8 * i) * 1024, k_off[i], soff);
      if (wave + 8 * i < L::V_BLOCKS)
        bwd_load_lds16(vrs, stage + L::K_BYTES + (wave + 8 * i) * 1024, v_off[i], soff);
    }
  };
  auto wait_loads = []() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's loads into LDS have landed
    __builtin_amdgcn_sched_barrier(0);
  };
  // Workgroup barrier that does not wait for loads still in flight (a release fence
  // would): lgkmcnt(0) completes this wave's LDS reads; the empty asm statements keep
  // the compiler from moving memory accesses across it.
  auto tile_barrier = []() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // Tile t on its stage; `next` (the other stage, free since the last barrier) first
  // receives tile t + 1.  The pointers are restrict-qualified because they never
  // overlap; that also tells the compiler the reads of `cur` need not wait for the
  // loads into `next`.
  auto tile_work = [&](const int t, unsigned char* __restrict__ next, const unsigned char* __restrict__ cur)
      __attribute__((always_inline)) {
    if (t + 1 < n_tiles) load_tile(next, t + 1);
    const unsigned char* ks_ = cur;
    const unsigned char* vs_ = cur + L::K_BYTES;
    const int k0 = t * kDqTile;
    const bool edge = (causal && k0 + kDqTile - 1 > first_q) || (k0 + kDqTile > len_b);
    // the tile in two 32-key halves, each: S^T, dP^T, dS^T, then its two 16-key chunks of dQ^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sacc, dpacc;
#pragma unroll
      for (int kd = 0; kd < D / 16; ++kd) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks_ + (kb * 32 + col) * L::KTS + (kd * 16 + h * 8) * 2);
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(vs_ + (kb * 32 + col) * L::VTS + (kd * 16 + h * 8) * 2);
        sacc = mfma32(a, qf[kd], kd == 0 ? f32x16{} : sacc);
        dpacc = mfma32(v, of[kd], kd == 0 ? f32x16{} : dpacc);
      }
      // masked entries take exp2(-inf) = 0; off the edge tiles every key is visible
      auto grads = [&](auto masked_tag) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float arg = fmaf(sacc[e], c2, -lc);
          if constexpr (decltype(masked_tag)::value) {
            const int kk = k0 + kb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
            const bool vis = (kk < len_b) & (!causal | (kk <= qi));
            arg = vis ? arg : -INFINITY;
          }
          dpacc[e] = fast_exp2(arg) * (dpacc[e] - drow);
        }
      };
      if (edge) grads(std::true_type{});
      else grads(std::false_type{});
      bf16x8 dsf[2];
#pragma unroll
      for (int c2_ = 0; c2_ < 2; ++c2_) {
        const int e0 = 8 * c2_;
        dsf[c2_] = pack_bf16x8(dpacc[e0], dpacc[e0 + 1], dpacc[e0 + 2], dpacc[e0 + 3], dpacc[e0 + 4],
                               dpacc[e0 + 5], dpacc[e0 + 6], dpacc[e0 + 7]);
      }
#pragma unroll
      for (int c2_ = 0; c2_ < 2; ++c2_)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 a = load_vt_operand(ks_, L::KTS, 2 * kb + c2_, db * 32, lane);
          dqacc[db] = mfma32(a, dsf[c2_], dqacc[db]);
        }
    }
  };
  auto stage_at = [&](int t) { return lds + (t & 1) * L::STAGE; };
  if (n_tiles > 0) {
    load_tile(stage_at(0), 0);
    wait_loads();
    tile_barrier();
  }
  for (int t = 0; t < n_tiles; ++t) {
    tile_work(t, stage_at(t + 1), stage_at(t));
    wait_loads();                 // tile t + 1 has landed in this wave's blocks
    tile_barrier();               // ... in every wave's; and every wave is done with tile t
  }

  if (row_valid) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = db * 32 + 8 * j + 4 * h;
        *reinterpret_cast<float4*>(p.dq + rrow * D + d0) =
            make_float4(dqacc[db][4 * j] * p.scale, dqacc[db][4 * j + 1] * p.scale, dqacc[db][4 * j + 2] * p.scale,
                        dqacc[db][4 * j + 3] * p.scale);
      }
  }
}

template <int D>
hipError_t launch_t(BwdParams prm, hipStream_t s) {
  const long long rows = (long long)prm.B * prm.h_q * prm.T;
  // With O 16-byte aligned the dQ kernel forms delta from its rows and runs first; the
  // dK/dV kernel, which reads delta for every row of its items, follows it.  Otherwise
  // a separate pass computes delta with element loads before both.
  prm.dq_delta = reinterpret_cast<uintptr_t>(prm.o) % 16 == 0 ? 1 : 0;
  hipError_t e = hipSuccess;
  if (!prm.dq_delta) {
    hipLaunchKernelGGL(bwd_delta_kernel<D>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, prm);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  static std::atomic<unsigned long long> dkdv_allowed{0}, dq_allowed{0};
  e = allow_dynamic_lds(reinterpret_cast<const void*>(bwd_dq_kernel<D>), DqLds<D>::TOTAL, dq_allowed);
  if (e != hipSuccess) return e;
  const long long n_dq = (long long)prm.B * prm.h_kv * prm.n_hchunks * prm.n_qblocks;
  hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)n_dq), dim3(kDqThreads), DqLds<D>::TOTAL, s, prm);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_kb = (prm.T + kKeyBlock - 1) / kKeyBlock;
  if constexpr (D == 128) {
    e = allow_dynamic_lds(reinterpret_cast<const void*>(bwd_dkdv16_kernel), Dkdv16Lds::TOTAL, dkdv_allowed);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dkdv16_kernel, dim3((unsigned)(prm.B * prm.h_kv * n_kb)), dim3(kDk16Threads),
                       Dkdv16Lds::TOTAL, s, prm);
  } else {
    e = allow_dynamic_lds(reinterpret_cast<const void*>(bwd_dkdv_kernel<D>), DkdvLds<D>::TOTAL, dkdv_allowed);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)(prm.B * prm.h_kv * n_kb)), dim3(kBwdThreads),
                       DkdvLds<D>::TOTAL, s, prm);
  }
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int B, int h_q, int T) { return (size_t)B * h_q * T * sizeof(float); }

hipError_t launch_backward_bf16(const BwdArgs& a, hipStream_t s) {
  BwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = a.o;
  p.d_o = static_cast<const uint16_t*>(a.d_o);
  p.lse = a.lse;
  p.delta = static_cast<float*>(a.workspace);
  p.dq = a.dq; p.dk = a.dk; p.dv = a.dv;
  p.kv_lens = a.kv_lens;
  p.B = a.B; p.h_q = a.h_q; p.h_kv = a.h_kv; p.r = a.h_q / a.h_kv; p.T = a.T;
  p.causal = a.causal; p.o_bf16 = a.o_bf16;
  int hp = 1;
  while (hp < kDqRows && p.r % (hp * 2) == 0) hp *= 2;
  p.hp = hp;
  p.P = kDqRows / hp;
  p.n_qblocks = (a.T + p.P - 1) / p.P;
  p.n_hchunks = p.r / hp;
  p.scale = a.scale;
  p.c = a.scale * kLog2e;
  const long long n_dq = (long long)a.B * a.h_kv * p.n_hchunks * p.n_qblocks;
  const long long n_kv = (long long)a.B * a.h_kv * ((a.T + kKeyBlock - 1) / kKeyBlock);
  if (n_dq > 0x7fffffffLL || n_kv > 0x7fffffffLL || (long long)a.B * a.h_q * a.T / 4 + 1 > 0x7fffffffLL)
    return hipErrorInvalidValue;
  return a.D == 128 ? launch_t<128>(p, s) : launch_t<64>(p, s);
}

}  // namespace gqa
