// Exact-attention backward for gfx950 (MI355X): preprocess, main, dQ convert.
//
// The backward recomputes P from Q, K and the forward's LSE instead of
// storing it (hotdry article, kernel-fusion section) and runs five bf16 MFMA
// products per K/V tile and query step (hotelren summary, sections 4.1-4.2):
//   S  = Q K^T              P  = exp2(S c - LSE log2 e)
//   dP = dO V^T             dS = P o (dP - Delta),  Delta_i = dO_i . O_i
//   dV += P^T dO            dK += dS^T Q            dQ += dS K
// dK and dV of a key tile are owned by one workgroup.  dQ has three modes
// (atomic and fixed-order accumulation: danialwang explainer, sections 05-06):
//   atomic        the main kernel also forms dQ += dS K for its key tile and
//                 adds it into an fp32 workspace with atomics;
//   stored dS     the main kernel writes its bf16 dS blocks to the workspace
//                 and a separate kernel owns each query tile, sums dS K over
//                 the key tiles in ascending order and writes dQ once;
//   recompute     like stored dS, but the dQ kernel recomputes S, dP and dS
//                 instead of reading them (small workspace).
// The two fixed-order modes use no atomics, so their results are
// bit-identical run to run.
//
// Layout choices.  S is computed with keys as the MFMA accumulator's column
// (lane) index.  Its accumulator registers are then, unchanged, the A operand
// of P^T dO and dS^T Q (a C-layout tile read as an A operand is its own
// transpose), which is the "compute the transposed form so the result is the
// next product's operand" idea of the danialwang explainer (section 05).  The
// B operands of those two products need 8 queries of one d per lane; they are
// read from the row-major Q and dO tiles with ds_read_b64_tr_b16.  dQ
// contracts over keys, so dS^T takes one trip through LDS and is read back
// with the same transposing read.
//
// Pipeline (main kernel): Q, dO, LSE*log2e and Delta of query step i+1 are
// copied from HBM straight into LDS (buffer_load ... lds) while step i
// computes; in atomic mode the dQ product of step i runs during step i+1,
// after the one barrier per step that publishes step i's dS^T.
#include <atomic>
#include <mutex>

#include "../../include/fa.h"
#include "common.hpp"
#include "kernels.hpp"

namespace fa {
namespace {

constexpr int kBwdBN = 128;    // keys per workgroup (32 per wave)
constexpr int kBwdWaves = 4;


struct BwdParams {
  int B, Hq, G, N;
  int nkb;         // key tiles per head
  int nqs;         // query steps per head
  float c;         // scale * log2(e)
  float scale;
  float* dq_acc;   // fp32 [B][Hq][N][D] (atomic mode)
  float* delta;    // fp32 [B][Hq][N]
  float* lse2;     // fp32 [B][Hq][N]
  char* ds;        // dS^T blocks (stored-dS mode), ds_head bytes per (b, hq) (packed: per hq)
  uint32_t ds_head;
  // Stored-dS mode with packed sequences: sequence b's blocks start at block
  // blk_off[b] of each head's region (B + 1 entries, clamped to its size).
  const int* blk_off;
  int hsplit;      // query-head parts per K/V head (warp-specialized kernel)
  float* kv_part;  // fp32 partial dK, dV when hsplit > 1
  int nb32;        // 32-row blocks per head, ceil(N / 32)
  // Variable length: cumulative sequence starts, the token count, and the
  // work list of this kernel (2 ints per item) with its length.
  const int* cu;
  int total;
  const int* items;
  const int* n_items;
};

// Geometry of one workgroup's sequence: its length, where its rows start in
// one head's matrix, and the distance between two heads (in rows).
struct SeqGeom {
  int N;
  size_t row0;   // first row of this sequence within a head
  size_t hstride;  // rows per head: N (dense) or total (variable length)
};

// dQ modes (the deterministic argument of the C ABI).
constexpr int kDqAtomic = 0;     // main kernel adds dS K into an fp32 buffer
constexpr int kDqStored = 1;     // main kernel stores dS; a fixed-order pass forms dS K
constexpr int kDqRecompute = 2;  // a fixed-order pass recomputes S, dP, dS and forms dS K

// Stored-dS layout: per (b, hq), the 32 x 32 dS^T block (query block qb32,
// key block kb32) at byte (qb32 * nb32 + kb32) * 2048.  Within a block, key
// row r's query positions 16u + 8h .. +8 are the 16-byte chunk 64u + 32h + r,
// and position p = 16u + 8h + i holds query 16u + 4h + (i & 3) + 8 (i >> 2)
// of the block (the order of the main kernel's MFMA A-operand registers,
// stored unchanged).

// ---------------------------------------------------------------------------
// Preprocess: Delta_i = sum_d dO[i,d] O[i,d] (fp32), LSE_i * log2(e), and
// (atomic mode) zero the dQ accumulator.  A row of D bf16 is read by D/8
// lanes (16 B each).
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ O,
                                                      const uint16_t* __restrict__ dO,
                                                      const float* __restrict__ LSE,
                                                      BwdParams p, int rows) {
  constexpr int LPR = D / 8;                 // lanes per row
  constexpr int RPB = 256 / LPR;             // rows per block
  const int tid = threadIdx.x;
  const int row = blockIdx.x * RPB + tid / LPR;
  const int c = tid % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *(const u32x4*)(O + (size_t)row * D + c * 8);
    const u32x4 b = *(const u32x4*)(dO + (size_t)row * D + c * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc += bf16_bits_to_float(a[j] & 0xffffu) * bf16_bits_to_float(b[j] & 0xffffu);
      acc += bf16_bits_to_float(a[j] >> 16) * bf16_bits_to_float(b[j] >> 16);
    }
    if (p.dq_acc) {
      float4* z = (float4*)(p.dq_acc + (size_t)row * D + c * 8);
      z[0] = make_float4(0.f, 0.f, 0.f, 0.f);
      z[1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && c == 0) {
    p.delta[row] = acc;
    p.lse2[row] = LSE[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// Atomic-mode backward kernel: dK, dV and each key tile's dQ contribution,
// added into an fp32 accumulator with atomics.  Workgroup =
// (batch, K/V head, key tile of 128); wave w owns keys 32w..32w+31 of the
// tile.  Query steps of QS = 4096 / D queries (32 for D = 128, 64 for D = 64)
// are walked from the last one down to the first that meets the tile's
// diagonal, for each of the G query heads.
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256, 1) void bwd_atomic_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, BwdParams p) {
  constexpr int BN = kBwdBN;
  constexpr int RB = D * 2;           // bytes per Q/dO/K/V row
  constexpr int KCH = D / 8;          // 16-byte chunks per row
  constexpr int QS = 4096 / D;        // queries per step
  constexpr int NQB = QS / 32;        // 32-query blocks per step
  constexpr int ND = D / 32;          // 32-wide d blocks
  constexpr int TB = QS * RB;         // bytes of one Q (or dO) step tile
  constexpr int NLD = TB / 1024 / kBwdWaves;  // 1 KiB direct loads per wave per tensor
  constexpr int DSB = BN * QS * 2;    // bytes of one dS^T buffer [key][query]
  constexpr int DSRB = QS * 2;        // bytes per dS^T row
  static_assert(NQB * ND == kBwdWaves, "one dQ output block per wave");
  static_assert(NLD >= 1, "step tile too small");

  // Per stage: Q tile, dO tile, 256 B of LSE*log2e, 256 B of Delta; then two
  // dS^T buffers.
  // Four stages: the step being finished (its LSE, Delta and the transposing
  // reads of its Q and dO), the next step (row reads of Q and dO for its S and
  // dP), and two more in flight, so a copy has two steps to land.  Each buffer
  // is its own array so the compiler can tell an in-flight copy from reads of
  // the others.
  constexpr int STAGE = 2 * TB + 512;
  __shared__ __attribute__((aligned(1024))) char stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[STAGE];
  __shared__ __attribute__((aligned(1024))) char stage2[STAGE];
  __shared__ __attribute__((aligned(1024))) char stage3[STAGE];
  __shared__ __attribute__((aligned(1024))) char dsbuf0[DSB];
  __shared__ __attribute__((aligned(1024))) char dsbuf1[DSB];

  const int Hkv = p.Hq / p.G;
  const int wg = blockIdx.x;
  int b, hk, kb;
  SeqGeom sg;
  if constexpr (VARLEN) {
    // Work list of (sequence, 128-key block), largest first; heads fastest.
    const int item = wg / Hkv;
    hk = wg % Hkv;
    if (item >= *p.n_items) return;
    b = p.items[2 * item];
    kb = p.items[2 * item + 1];
    const int s0 = min(max(p.cu[b], 0), p.total);
    sg.N = min(max(p.cu[b + 1] - s0, 0), p.total - s0);
    sg.row0 = (size_t)s0;
    sg.hstride = (size_t)p.total;
  } else {
    const int bhk = wg % (p.B * Hkv);
    kb = wg / (p.B * Hkv);
    b = bhk / Hkv;
    hk = bhk % Hkv;
    sg.N = p.N;
    sg.row0 = 0;
    sg.hstride = (size_t)p.N;
  }
  // Head h of batch b starts at row (b H + h) hstride + row0 (dense: b is the
  // batch; variable length: b = 0 in the head index, the sequence is row0).
  const int bq = VARLEN ? 0 : b;
  const int N = sg.N;
  const int nqs = (N + QS - 1) / QS;
  const int k0 = kb * BN;

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int n = lane & 31, h = lane >> 5;
  const int kw = k0 + 32 * wave;     // this wave's first key (uniform)
  const int key = kw + n;            // key this lane carries as MFMA column

  const uint32_t head_bytes = (uint32_t)((size_t)N * D * 2);   // one head's rows of this sequence
  const size_t kv_head = (((size_t)bq * Hkv + hk) * sg.hstride + sg.row0) * D;
  const rsrc_t kr = make_rsrc_uniform(K + kv_head, head_bytes);
  const rsrc_t vr = make_rsrc_uniform(V + kv_head, head_bytes);

  // Resident B operands for S = Q K^T and dP = dO V^T (k = d); keys past N
  // read as zero.
  bf16x8 kB[D / 16], vB[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    kB[t] = as_bf16x8(buf_load16(kr, (uint32_t)(key * RB + 32 * t + 16 * h)));
    vB[t] = as_bf16x8(buf_load16(vr, (uint32_t)(key * RB + 32 * t + 16 * h)));
  }
  // Resident B operand of this wave's dQ block (k = the tile's 128 keys):
  // lane (d, h) holds K[k0 + 16t + 8(i/4) + 4h + i%4][d] in slot i, matching
  // the transposing read of dS^T.
  const int dq_qb = wave / ND, dq_db = wave % ND;
  bf16x8 kT[BN / 16];
  {
    const int d = 32 * dq_db + n;
    const uint16_t* Kh = K + kv_head;
#pragma unroll
    for (int t = 0; t < BN / 16; ++t) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r0 = k0 + 16 * t + 8 * (j >> 1) + 4 * h + 2 * (j & 1);
        const uint32_t lo = (r0 < N) ? Kh[(size_t)r0 * D + d] : 0u;
        const uint32_t hi = (r0 + 1 < N) ? Kh[(size_t)(r0 + 1) * D + d] : 0u;
        w[j] = lo | (hi << 16);
      }
      kT[t] = as_bf16x8(w);
    }
  }

  f32x16 dk_acc[ND], dv_acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk_acc[i][r] = 0.f;
      dv_acc[i][r] = 0.f;
    }

  // ---- per-lane LDS offsets ------------------------------------------------
  // Direct loads: load s of this wave fills chunks g = (s*4 + wave)*64 + lane
  // of a step tile (row g / KCH, physical chunk g % KCH holds logical chunk
  // (g % KCH) ^ f(row)).
  uint32_t ld_off[NLD];
#pragma unroll
  for (int s = 0; s < NLD; ++s) {
    const int g = (s * kBwdWaves + wave) * 64 + lane;
    const int row = g / KCH, pc = g % KCH;
    ld_off[s] = (uint32_t)(row * RB + ((pc ^ tile_swz<D>(row)) * 16));
  }
  // Row-major A operand (Q of S, dO of dP): row 32 qb + n, logical chunk 2t+h.
  uint32_t a_off[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) a_off[t] = (uint32_t)(n * RB + (((2 * t + h) ^ tile_swz<D>(n)) * 16));
  // Transposing B-operand reads of Q / dO (queries 32 qb + 16 u + 8 rd + 4 h +
  // 0..3 of column d = 32 db + n): lane j of 16-lane group gq points at row
  // 8 rd + 4 h + j/4 and d = 32 db + 16 (gq & 1) + 4 (j & 3).
  const int tj = lane & 15, gq = lane >> 4;
  uint32_t tr_off[ND][2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int row = 8 * rd + 4 * h + (tj >> 2);
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const int c = 4 * db + 2 * (gq & 1) + ((tj & 3) >> 1);
      tr_off[db][rd] = (uint32_t)(row * RB + ((c ^ tile_swz<D>(row)) * 16) + (tj & 1) * 8);
    }
  }
  // dS^T [key][query] (rows of DSRB bytes): 16-byte chunk c of row r sits at
  // chunk c ^ fd(r), its two 8-byte halves swapped when fh(r) = 1.  Both
  // are XORs of row bits chosen so that the writer (16 or 32 consecutive
  // rows, one 8-byte half each) and the transposing reader (4 consecutive
  // rows, 2 or 4 chunks each) touch every bank equally, whether the LDS
  // serves 16 or 32 lanes at a time from 32 or 64 banks: the writer's row
  // bits map one to one onto the 8-byte positions of each 128- or 256-byte
  // bank window, and rows sharing a window on the reader's side get
  // disjoint chunk groups.
  auto fd = [](int r) {
    return QS == 32 ? (((((r >> 1) ^ (r >> 3)) & 1) << 1) | ((r >> 2) & 1))
                    : ((((r >> 1) & 1) << 2) | (((r ^ (r >> 2)) & 1) << 1) | ((r >> 3) & 1));
  };
  auto fh = [](int r) { return QS == 32 ? (((r >> 3) ^ (r >> 4)) & 1) : (((r >> 2) ^ (r >> 4)) & 1); };
  // Writer: lane (key 32 wave + n) stores 4 consecutive queries 32 qb + 8 g + 4 h.
  // Reader (A operand of dQ): lane j of group gq points at key row
  // 16 t + 8 rd + 4 h + j/4 and query 32 dq_qb + 16 (gq & 1) + 4 (j & 3);
  // the swizzle depends on the row's bits 3 and 4, so the offsets are kept
  // per (t & 1, rd).
  uint32_t dsr_off[2][2];
#pragma unroll
  for (int tp = 0; tp < 2; ++tp)
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int row = 16 * tp + 8 * rd + 4 * h + (tj >> 2);
      const int col = 32 * dq_qb + 16 * (gq & 1) + 4 * (tj & 3);
      dsr_off[tp][rd] =
          (uint32_t)(row * DSRB + (((col >> 3) ^ fd(row)) * 16) + ((((col >> 2) & 1) ^ fh(row)) * 8));
    }
  const int ds_wrow = 32 * wave + n;

  // ---- step schedule -------------------------------------------------------
  // Steps walk (head g, query step qs) with qs descending from the last step
  // to the first that meets the tile's diagonal, then on to the next of the G
  // query heads.  Two cursors follow it with scalar increments only: the next
  // step to copy in and the step being finished.
  const int qs_first = CAUSAL ? (k0 / QS) : 0;
  const int per_head = max(nqs - qs_first, 0);
  const int nsteps = p.G * per_head;
  const int hq0 = hk * p.G;
  const uint32_t lse_head_bytes = (uint32_t)N * 4u;       // range of one head's row constants
  const size_t q_hstride = sg.hstride * D * 2;             // bytes between two query heads
  const size_t l_hstride = sg.hstride * 4;
  const size_t qrow0 = ((size_t)bq * p.Hq + hq0) * sg.hstride + sg.row0;  // row of head hq0

  // Copy cursor: query step and the per-head base addresses of Q, dO, LSE, Delta.
  int iss_qs = nqs - 1;
  const char* iss_q = (const char*)(Q + qrow0 * D);
  const char* iss_do = (const char*)(dO + qrow0 * D);
  const char* iss_l = (const char*)(p.lse2 + qrow0);
  const char* iss_d = (const char*)(p.delta + qrow0);
  auto issue_next = [&](char* st) {
    const uint32_t base = (uint32_t)iss_qs * (uint32_t)TB;
    const uint32_t left = head_bytes - base;  // qs < nqs, so base < head_bytes
    const rsrc_t qrr = make_rsrc_uniform(iss_q + base, left);
    const rsrc_t dor = make_rsrc_uniform(iss_do + base, left);
#pragma unroll
    for (int s = 0; s < NLD; ++s) {
      lds_dma16(qrr, (lds_void*)(st + (s * kBwdWaves + wave) * 1024), ld_off[s]);
      lds_dma16(dor, (lds_void*)(st + TB + (s * kBwdWaves + wave) * 1024), ld_off[s]);
    }
    const uint32_t rbase = (uint32_t)iss_qs * (uint32_t)(QS * 4);
    const uint32_t rleft = lse_head_bytes - rbase;
    if (wave == 0) lds_dma4(make_rsrc_uniform(iss_l + rbase, rleft), (lds_void*)(st + 2 * TB), lane * 4);
    if (wave == 1) lds_dma4(make_rsrc_uniform(iss_d + rbase, rleft), (lds_void*)(st + 2 * TB + 256), lane * 4);
    if (--iss_qs < qs_first) {
      iss_qs = nqs - 1;
      iss_q += q_hstride;
      iss_do += q_hstride;
      iss_l += l_hstride;
      iss_d += l_hstride;
    }
  };
  // Cursor of the step being finished (query step and head offset g).
  int cur_qs = nqs - 1, cur_g = 0;
  int prev_qs = 0, prev_g = 0;  // the step before it (atomic dQ)
  auto advance_cur = [&]() {
    prev_qs = cur_qs;
    prev_g = cur_g;
    if (--cur_qs < qs_first) {
      cur_qs = nqs - 1;
      ++cur_g;
    }
  };
  // Wait until at most one step's copies (the newest) are outstanding: waves 0
  // and 1 issue one extra row-constant copy per step.
  auto wait_all_but_one_step = [&]() {
    if (wave < 2) wait_vmcnt<2 * NLD + 1>();
    else wait_vmcnt<2 * NLD>();
  };

  // dQ block of the step at (head offset g, query step qs), whose dS^T is in dsb.
  auto dq_step = [&](int g, int qs, const char* dsb) {
    const int hq = hq0 + g;
    const int q0 = qs * QS;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int t = 0; t < BN / 16; ++t) {
      const char* base = dsb + (16 * (t & ~1)) * DSRB;
      const u32x2 lo = lds_read_tr16((const lds_void*)(base + dsr_off[t & 1][0]));
      const u32x2 hi = lds_read_tr16((const lds_void*)(base + dsr_off[t & 1][1]));
      const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
      acc = mfma32(as_bf16x8(a), kT[t], acc);
    }
    // acc register r: query q0 + 32 dq_qb + 8(r/4) + 4h + r%4, d = 32 dq_db + n.
    const size_t qh = ((size_t)bq * p.Hq + hq) * sg.hstride + sg.row0;
    float* dqh = p.dq_acc + qh * D;
    const int qrow0 = q0 + 32 * dq_qb + 4 * h;
    const int d = 32 * dq_db + n;
    const rsrc_t dqr = make_rsrc_uniform(dqh, (uint32_t)((size_t)N * D * 4));
#pragma unroll
    for (int r = 0; r < 16; ++r)
      buf_atomic_add(dqr, (uint32_t)(((qrow0 + 8 * (r >> 2) + (r & 3)) * D + d) * 4), acc[r]);
  };

  // S and dP of one step (A operands Q, dO by row reads of its stage).
  auto compute_sdp = [&](const char* st, f32x16 (&sv)[NQB], f32x16 (&dv)[NQB]) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sv[qb][r] = 0.f;
        dv[qb][r] = 0.f;
      }
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const bf16x8 qa = as_bf16x8(*(const u32x4*)(st + qb * 32 * RB + a_off[t]));
        const bf16x8 da = as_bf16x8(*(const u32x4*)(st + TB + qb * 32 * RB + a_off[t]));
        sv[qb] = mfma32(qa, kB[t], sv[qb]);
        dv[qb] = mfma32(da, vB[t], dv[qb]);
      }
    }
  };

  // One step i, software-pipelined: while the VALU forms P(i) and dS(i), the
  // MFMA unit computes S(i+1) and dP(i+1); then dV, dK take step i's products.
  // sv/dv hold S(i), dP(i); sn/dn receive S(i+1), dP(i+1).
  auto body = [&](int i, const char* cur, const char* nxt, char* ld, char* dsw,
                  const char* dsprev, f32x16 (&sv)[NQB], f32x16 (&dv)[NQB], f32x16 (&sn)[NQB],
                  f32x16 (&dn)[NQB], const f32x4 (&lc)[NQB][4], const f32x4 (&dc)[NQB][4],
                  f32x4 (&ln)[NQB][4], f32x4 (&dln)[NQB][4]) {
    // Step i+1 must be in LDS.  __syncthreads' fence then drains the rest as
    // well (direct-to-LDS copies count in vmcnt): this kernel's atomics do
    // not complete in order with its copies, so it does not keep copies in
    // flight across the barrier.
    if (i + 2 < nsteps) wait_all_but_one_step();
    else wait_vmcnt<0>();
    __syncthreads();  // step i+1 visible to all; step i-1's stage and dS^T free
    if (i + 3 < nsteps) issue_next(ld);
    if (i > 0) dq_step(prev_g, prev_qs, dsprev);

    const int q0 = cur_qs * QS;
    // S(i) and dP(i) are read by the VALU below: move them to VGPRs here, so
    // that the masked and unmasked paths join in VGPRs (otherwise the masked
    // values go back to the accumulator registers and are read out again).
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      pin(sv[qb]);
      pin(dv[qb]);
    }
    // Causal mask of step i, only near the diagonal: S = -inf where key > query.
    // Register r of block qb holds query q0 + 32qb + 8(r/4) + 4h + r%4.
    // Padding keys (key >= N, rows read as zero) are masked too: their score 0
    // can exceed every real score and overflow P.
    if ((CAUSAL && (q0 < kw + 31)) || (kw + 32 > N)) {
      keep_branch();
      const int lim = (key >= N) ? 1 << 30 : (CAUSAL ? key - q0 - 4 * h : -1);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * qb + 8 * (r >> 2) + (r & 3) < lim) sv[qb][r] = -__builtin_inff();
    }

    // The issue order below is fixed by hand (sched_barrier fences): the
    // MFMA unit runs one instruction at a time, in program order, so each
    // matrix instruction is followed by the VALU work that should run under it.
    // Phase A: the 16 S(i+1)/dP(i+1) MFMAs (always computed, on a stale stage
    // after the last step, so the phase has no branch), each pair followed by
    // 2 NQB elements of P(i) = exp2(S c - LSE log2 e), dS(i) = P (dP - Delta).
    // Phase B: the dV += P^T dO, dK += dS^T Q MFMAs.  LDS operands of both
    // phases form one stream read PD pairs ahead of their MFMAs; step i+1's
    // LSE and Delta are read during phase B.
    constexpr int T = D / 16;
    constexpr int NPAIR = NQB * T;         // S/dP MFMA pairs (8 for D = 64, 128)
    constexpr int EPP = 16 * NQB / NPAIR;  // elements per lane per pair
    constexpr int NB = NQB * ND * 2;       // dV/dK MFMA pairs
    constexpr int PD = 2;                  // operand prefetch distance, in pairs
    const char* qs_l = cur;
    const char* dos_l = cur + TB;
    // LSE * log2 e and Delta of step i: read by the previous step when one
    // block per step (D = 128); read here when two (D = 64, where a second
    // register set would not fit).
    constexpr bool EARLY_ROWC = NQB == 1;
    f32x4 lcur[NQB][4], dcur[NQB][4];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        if constexpr (EARLY_ROWC) {
          lcur[qb][r4] = lc[qb][r4];
          dcur[qb][r4] = dc[qb][r4];
        } else {
          lcur[qb][r4] = *(const f32x4*)((const float*)(cur + 2 * TB) + 32 * qb + 8 * r4 + 4 * h);
          dcur[qb][r4] = *(const f32x4*)((const float*)(cur + 2 * TB + 256) + 32 * qb + 8 * r4 + 4 * h);
        }
      }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sn[qb][r] = 0.f;
        dn[qb][r] = 0.f;
      }
    // Operand stream: c < NPAIR is phase A pair c (row reads of Q, dO of step
    // i+1); c >= NPAIR is phase B pair c - NPAIR = (qb, u, db), db fastest so
    // that consecutive MFMAs never accumulate into the same registers
    // (transposing reads of dO, Q of step i).
    bf16x8 opA[NPAIR + NB], opB[NPAIR + NB];
    auto fetch = [&](int c) {
      if (c < NPAIR) {
        const int qb1 = c / T, t1 = c % T;
        opA[c] = as_bf16x8(*(const u32x4*)(nxt + qb1 * 32 * RB + a_off[t1]));
        opB[c] = as_bf16x8(*(const u32x4*)(nxt + TB + qb1 * 32 * RB + a_off[t1]));
      } else if (c < NPAIR + NB) {
        const int jb = c - NPAIR;
        const int qb = jb / (2 * ND), u = (jb / ND) & 1, db = jb % ND;
        const int roff = (32 * qb + 16 * u) * RB;
        const u32x2 olo = lds_read_tr16((const lds_void*)(dos_l + roff + tr_off[db][0]));
        const u32x2 ohi = lds_read_tr16((const lds_void*)(dos_l + roff + tr_off[db][1]));
        const u32x2 qlo = lds_read_tr16((const lds_void*)(qs_l + roff + tr_off[db][0]));
        const u32x2 qhi = lds_read_tr16((const lds_void*)(qs_l + roff + tr_off[db][1]));
        opA[c] = as_bf16x8(u32x4{olo[0], olo[1], ohi[0], ohi[1]});
        opB[c] = as_bf16x8(u32x4{qlo[0], qlo[1], qhi[0], qhi[1]});
      }
    };
#pragma unroll
    for (int c = 0; c < PD; ++c) fetch(c);
    bf16x8 pa[NQB][2], dsa[NQB][2];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NPAIR; ++j) {
      const int qb = j / T, t = j % T;
      fetch(j + PD);
      sn[qb] = mfma32(opA[j], kB[t], sn[qb]);
      dn[qb] = mfma32(opB[j], vB[t], dn[qb]);
#pragma unroll
      for (int e = j * EPP; e < (j + 1) * EPP; ++e) {
        const int eq = e / 16, r = e % 16;
        const float pv = exp2_hw(__builtin_fmaf(sv[eq][r], p.c, -lcur[eq][r >> 2][r & 3]));
        sv[eq][r] = pv;
        dv[eq][r] = pv * (dv[eq][r] - dcur[eq][r >> 2][r & 3]);
        if ((r & 7) == 7) {
          const int u = r >> 3;
          u32x4 w1, w2;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            w1[m] = pack_bf16x2(sv[eq][8 * u + 2 * m], sv[eq][8 * u + 2 * m + 1]);
            w2[m] = pack_bf16x2(dv[eq][8 * u + 2 * m], dv[eq][8 * u + 2 * m + 1]);
          }
          pa[eq][u] = as_bf16x8(w1);
          dsa[eq][u] = as_bf16x8(w2);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // Phase B.
    const float* lse_n = (const float*)(nxt + 2 * TB);
    const float* dlt_n = (const float*)(nxt + 2 * TB + 256);
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
      const int qb = jb / (2 * ND), u = (jb / ND) & 1, db = jb % ND;
      fetch(NPAIR + jb + PD);
      dv_acc[db] = mfma32(pa[qb][u], opA[NPAIR + jb], dv_acc[db]);
      dk_acc[db] = mfma32(dsa[qb][u], opB[NPAIR + jb], dk_acc[db]);
      // Step i+1's LSE * log2 e and Delta for this lane's queries.
      if (EARLY_ROWC && jb < NQB * 4) {
        const int lq = jb / 4, r4 = jb % 4;
        ln[lq][r4] = *(const f32x4*)(lse_n + 32 * lq + 8 * r4 + 4 * h);
        dln[lq][r4] = *(const f32x4*)(dlt_n + 32 * lq + 8 * r4 + 4 * h);
      }
      // dS^T -> LDS: lane (key 32 wave + n) writes queries 32qb + 8g + 4h .. +4.
      if (db == 0 && u == 0) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int col = 32 * qb + 8 * g4 + 4 * h;
          const u32x4 dsw4 = as_u32x4(dsa[qb][g4 >> 1]);
          u32x2 w;
          w[0] = dsw4[(g4 & 1) * 2];
          w[1] = dsw4[(g4 & 1) * 2 + 1];
          *(u32x2*)(dsw + ds_wrow * DSRB + (((col >> 3) ^ fd(ds_wrow)) * 16) +
                    ((((col >> 2) & 1) ^ fh(ds_wrow)) * 8)) = w;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    advance_cur();
  };

  f32x16 sA[NQB], dA[NQB], sB[NQB], dB[NQB];
  // LSE * log2 e and Delta of the step being finished (set A or B, alternating
  // like the S/dP sets; each body reads the next step's into the other set).
  f32x4 lA[NQB][4], dlA[NQB][4], lB[NQB][4], dlB[NQB][4];
  if (nsteps > 0) {
    issue_next(stage0);
    if (nsteps > 1) issue_next(stage1);
    if (nsteps > 2) issue_next(stage2);
    // Step 0 complete: with three steps issued, two may still be in flight.
    if (nsteps > 2) {
      if (wave < 2) wait_vmcnt<4 * NLD + 2>();
      else wait_vmcnt<4 * NLD>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    compute_sdp(stage0, sA, dA);
    if constexpr (NQB == 1)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        lA[qb][r4] = *(const f32x4*)((const float*)(stage0 + 2 * TB) + 32 * qb + 8 * r4 + 4 * h);
        dlA[qb][r4] = *(const f32x4*)((const float*)(stage0 + 2 * TB + 256) + 32 * qb + 8 * r4 + 4 * h);
      }
  }
  // Stages rotate with period 4, S/dP register sets and dS^T buffers with
  // period 2.  The main loop has no bounds checks between bodies, so the
  // register sets keep their places; the tail checks each step.
  int i = 0;
  for (; i + 4 <= nsteps; i += 4) {
    body(i, stage0, stage1, stage3, dsbuf0, dsbuf1, sA, dA, sB, dB, lA, dlA, lB, dlB);
    body(i + 1, stage1, stage2, stage0, dsbuf1, dsbuf0, sB, dB, sA, dA, lB, dlB, lA, dlA);
    body(i + 2, stage2, stage3, stage1, dsbuf0, dsbuf1, sA, dA, sB, dB, lA, dlA, lB, dlB);
    body(i + 3, stage3, stage0, stage2, dsbuf1, dsbuf0, sB, dB, sA, dA, lB, dlB, lA, dlA);
  }
  if (i < nsteps) body(i, stage0, stage1, stage3, dsbuf0, dsbuf1, sA, dA, sB, dB, lA, dlA, lB, dlB);
  if (i + 1 < nsteps)
    body(i + 1, stage1, stage2, stage0, dsbuf1, dsbuf0, sB, dB, sA, dA, lB, dlB, lA, dlA);
  if (i + 2 < nsteps)
    body(i + 2, stage2, stage3, stage1, dsbuf0, dsbuf1, sA, dA, sB, dB, lA, dlA, lB, dlB);
  if (nsteps > 0) {
    __syncthreads();
    dq_step(prev_g, prev_qs, ((nsteps - 1) & 1) ? dsbuf1 : dsbuf0);
  }

  // ---- dK (scaled) and dV of this wave's 32 keys ----------------------------
  // Accumulator register r of d-block db: key kw + 8(r/4) + 4h + r%4, d = 32db + n.
  uint16_t* dKh = dK + kv_head;
  uint16_t* dVh = dV + kv_head;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int krow = kw + 8 * (r >> 2) + 4 * h + (r & 3);
      if (krow < N) {
        const size_t off = (size_t)krow * D + 32 * db + n;
        dKh[off] = (uint16_t)(pack_bf16x2(dk_acc[db][r] * p.scale, 0.f) & 0xffffu);
        dVh[off] = (uint16_t)(pack_bf16x2(dv_acc[db][r], 0.f) & 0xffffu);
      }
    }
}

// ---------------------------------------------------------------------------
// Warp-specialized main backward kernel, D = 64 or 128 (dQ modes stored and
// recompute; dense or packed sequences).  Same work item as bwd_atomic_kernel -- (batch, K/V head, 128-key
// tile), every query step of every query head of the group -- with 8 waves in
// two roles over the same step tiles:
//   score waves 0..3 (keys 32 w): the MFMA unit forms S, dP of step i+1 while
//     the VALU forms P(i) = exp2(S c - LSE log2 e) and dS(i) = P (dP - Delta);
//     P(i) and dS(i) go to LDS in MFMA operand order (and, stored mode, dS(i)
//     to the workspace);
//   gradient waves 4..7 (one product each over all 128 keys, half of the d
//     range: waves 4, 5 dV += P^T dO, waves 6, 7 dK += dS^T Q) of step i-1,
//     P and dS from the score waves' LDS slots, dO^T and Q^T by transposing
//     reads of the step tile.
// Waves are dealt to the 4 SIMDs round-robin, so waves w and w + 4 share one:
// the exp2-heavy score stream and the MFMA-only gradient stream run side by
// side, and each role needs about half the registers of the single-role
// kernel, which is what lets two waves live on a SIMD.  One barrier per step.
// Step tiles rotate through six stages: step i-1 (transposing reads), i (its
// LSE and Delta), i+1 (row reads), i+2 .. i+4 (copies in flight; the step
// barrier does not drain them, and the gradient waves wait for exactly the
// copies that must be complete).  In the stored-dS mode at D = 128 (PREF)
// step i+2 is complete one step earlier, and the score waves read its first
// operands and step i+1's row constants before the next barrier, so their
// products start right after it (2.5% faster there with cached dS stores,
// equal with non-temporal ones; the recompute mode measured 1.8% slower with
// it, and the stored mode at D = 64 1.3% slower, so they keep the later
// reads).  Only the gradient waves copy step tiles in; only the score waves
// store dS, each half block as soon as it is packed.
template <int D, bool CAUSAL, int DQM, bool VARLEN>
__global__ __launch_bounds__(512, 1) void bwd_ws_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, BwdParams p) {
  static_assert(D == 64 || D == 128, "D = 64 or 128");
  constexpr int NW = 8;
  constexpr int BN = kBwdBN;
  constexpr int RB = D * 2;
  constexpr int KCH = D / 8;
  constexpr int QS = 32;              // queries per step
  constexpr int ND = D / 32;          // 32-wide d blocks
  constexpr int T = D / 16;           // k-steps of S and dP
  constexpr int EPJ = 16 / T;         // elements of P, dS formed per S/dP MFMA pair
  constexpr int TB = QS * RB;         // bytes of one Q (or dO) step tile
  constexpr int NLD = TB / 1024 / 4;  // 1 KiB direct loads per gradient wave and tensor
  constexpr bool STORE_DS = DQM == kDqStored;
  constexpr bool PREF = STORE_DS && D == 128;  // score-wave reads ahead of the barrier
  static_assert(NLD >= 1, "step tile too small");
  static_assert(DQM != kDqAtomic, "atomic dQ uses bwd_atomic_kernel");
  constexpr int STAGE = 2 * TB + 512;  // Q, dO, 256 B LSE * log2 e, 256 B Delta
  constexpr int PSLOT = 4 * 4096;      // P, dS of the 4 score waves
  __shared__ __attribute__((aligned(1024))) char st0[STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[STAGE];
  __shared__ __attribute__((aligned(1024))) char st3[STAGE];
  __shared__ __attribute__((aligned(1024))) char st4[STAGE];
  __shared__ __attribute__((aligned(1024))) char st5[STAGE];
  __shared__ __attribute__((aligned(1024))) char pb0[PSLOT];
  __shared__ __attribute__((aligned(1024))) char pb1[PSLOT];

  const int Hkv = p.Hq / p.G;
  const int wg = blockIdx.x;
  // Work item: (batch, K/V head, part hs of its G query heads, key tile);
  // key tiles vary slowest so the longest causal items start first.
  // Variable length: (sequence, key tile) from the list sorted largest
  // first, heads fastest, one part; a sequence's rows start at cu_seqlens[b]
  // in every head's [total][D] matrix.
  const int BHkv = p.B * Hkv;
  int b, hk, kb, hs, bhk;
  SeqGeom sg;
  if constexpr (VARLEN) {
    const int item = wg / Hkv;
    hk = wg % Hkv;
    if (item >= *p.n_items) return;  // whole workgroup: the grid is sized for the worst case
    b = p.items[2 * item];
    kb = p.items[2 * item + 1];
    hs = 0;
    bhk = hk;
    const int s0 = min(max(p.cu[b], 0), p.total);
    sg.N = min(max(p.cu[b + 1] - s0, 0), p.total - s0);
    sg.row0 = (size_t)s0;
    sg.hstride = (size_t)p.total;
  } else {
    bhk = wg % BHkv;
    hs = (wg / BHkv) % p.hsplit;
    kb = wg / BHkv / p.hsplit;
    b = bhk / Hkv;
    hk = bhk % Hkv;
    sg.N = p.N;
    sg.row0 = 0;
    sg.hstride = (size_t)p.N;
  }
  const int bq = VARLEN ? 0 : b;       // batch index in the head arithmetic
  const int gs = p.G / (VARLEN ? 1 : p.hsplit);  // query heads this workgroup walks
  const int N = sg.N;
  const int nqs = (N + QS - 1) / QS;
  const int k0 = kb * BN;

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const bool grad = wave >= 4;
  const int kwave = wave & 3;
  const int n = lane & 31, h = lane >> 5;
  const int kw = k0 + 32 * kwave;    // first key of this wave's 32 (uniform)
  const int key = kw + n;
  const uint32_t head_bytes = (uint32_t)((size_t)N * D * 2);
  const size_t kv_head = (((size_t)bq * Hkv + hk) * sg.hstride + sg.row0) * D;

  // ---- step copies (gradient waves only) ----------------------------------
  // The score waves issue no loads in the loop, so their only memory traffic,
  // the stored-dS writes, never delays a wait for a copy: vmcnt counts loads
  // and stores together, and a store can take long to be acknowledged.
  // Load s of gradient wave k fills chunks g = (s*4 + k)*64 + lane of a step
  // tile (row g / KCH, physical chunk g % KCH holding logical chunk
  // (g % KCH) ^ f(row)).
  uint32_t ld_off[NLD];
#pragma unroll
  for (int s = 0; s < NLD; ++s) {
    const int g = (s * 4 + kwave) * 64 + lane;
    const int row = g / KCH, pc = g % KCH;
    ld_off[s] = (uint32_t)(row * RB + ((pc ^ tile_swz<D>(row)) * 16));
  }
  const int qs_first = CAUSAL ? (k0 / QS) : 0;
  const int per_head = max(nqs - qs_first, 0);
  const int nsteps = gs * per_head;
  const int hq0 = hk * p.G + hs * gs;
  const uint32_t lse_head_bytes = (uint32_t)N * 4u;
  const size_t q_hstride = sg.hstride * D * 2;
  const size_t l_hstride = sg.hstride * 4;
  const size_t qrow0 = ((size_t)bq * p.Hq + hq0) * sg.hstride + sg.row0;
  int iss_qs = nqs - 1;
  const char* iss_q = (const char*)(Q + qrow0 * D);
  const char* iss_do = (const char*)(dO + qrow0 * D);
  const char* iss_l = (const char*)(p.lse2 + qrow0);
  const char* iss_d = (const char*)(p.delta + qrow0);
  auto issue_next = [&](char* st) {
    const uint32_t base = (uint32_t)iss_qs * (uint32_t)TB;
    const uint32_t left = head_bytes - base;
    const rsrc_t qrr = make_rsrc_uniform(iss_q + base, left);
    const rsrc_t dor = make_rsrc_uniform(iss_do + base, left);
#pragma unroll
    for (int s = 0; s < NLD; ++s) {
      lds_dma16(qrr, (lds_void*)(st + (s * 4 + kwave) * 1024), ld_off[s]);
      lds_dma16(dor, (lds_void*)(st + TB + (s * 4 + kwave) * 1024), ld_off[s]);
    }
    const uint32_t rbase = (uint32_t)iss_qs * (uint32_t)(QS * 4);
    const uint32_t rleft = lse_head_bytes - rbase;
    if (wave == 4) lds_dma4(make_rsrc_uniform(iss_l + rbase, rleft), (lds_void*)(st + 2 * TB), lane * 4);
    if (wave == 5) lds_dma4(make_rsrc_uniform(iss_d + rbase, rleft), (lds_void*)(st + 2 * TB + 256), lane * 4);
    if (--iss_qs < qs_first) {
      iss_qs = nqs - 1;
      iss_q += q_hstride;
      iss_do += q_hstride;
      iss_l += l_hstride;
      iss_d += l_hstride;
    }
  };
  // Gradient waves before barrier i: the copies of steps up to i+1 (PREF:
  // i+2) complete, the later ones issued so far (up to step i+3) may still be
  // in flight (waves 4 and 5 issue one extra row-constant copy per step;
  // loads complete in order).
  auto wait_step = [&](int i) {
    if (!PREF && i + 3 < nsteps) {
      if (wave < 6) wait_vmcnt<2 * (2 * NLD + 1)>();
      else wait_vmcnt<2 * (2 * NLD)>();
    } else if (i + (PREF ? 3 : 2) < nsteps) {
      if (wave < 6) wait_vmcnt<2 * NLD + 1>();
      else wait_vmcnt<2 * NLD>();
    } else {
      wait_vmcnt<0>();
    }
  };

  // Score waves: resident B operands of S = Q K^T and dP = dO V^T (keys past
  // N read as 0).
  bf16x8 kB[T], vB[T];
  if (!grad) {
    const rsrc_t kr = make_rsrc_uniform(K + kv_head, head_bytes);
    const rsrc_t vr = make_rsrc_uniform(V + kv_head, head_bytes);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      kB[t] = as_bf16x8(buf_load16(kr, (uint32_t)(key * RB + 32 * t + 16 * h)));
      vB[t] = as_bf16x8(buf_load16(vr, (uint32_t)(key * RB + 32 * t + 16 * h)));
    }
  }
  if (nsteps > 0 && grad) {
    issue_next(st0);
    if (nsteps > 1) issue_next(st1);
    if (nsteps > 2) issue_next(st2);
    if (nsteps > 3) issue_next(st3);
    // Step 0 (PREF: steps 0 and 1) complete; the later ones may be in flight.
    if (!PREF && nsteps > 3) {
      if (wave < 6) wait_vmcnt<3 * (2 * NLD + 1)>();
      else wait_vmcnt<3 * (2 * NLD)>();
    } else if (PREF && nsteps > 3) {
      if (wave < 6) wait_vmcnt<2 * (2 * NLD + 1)>();
      else wait_vmcnt<2 * (2 * NLD)>();
    } else {
      wait_vmcnt<0>();
    }
  }
  lds_barrier();

  if (!grad) {
    // ======================= score waves =======================
    // Row-major A operand (Q of S, dO of dP): row n, logical chunk 2t + h.
    uint32_t a_off[T];
#pragma unroll
    for (int t = 0; t < T; ++t) a_off[t] = (uint32_t)(n * RB + (((2 * t + h) ^ tile_swz<D>(n)) * 16));

    int cur_qs = nqs - 1, cur_g = 0;
    // Stored-dS mode: half u of this wave's dS^T block of the current step
    // goes out as soon as it is packed (spread over the step; these waves
    // issue no loads, so no wait ever covers the stores).  Lane (key n, half
    // h) holds positions 16u + 8h .. +8 of row n, stored at byte
    // 1024u + 16 lane of the block (whole cache lines per store); a block that
    // does not exist (padding rows, or above the diagonal under causal) gets
    // an offset past the end of the head's range and the store is dropped.
    // Packed sequences: the sequence's own grid of ceil(N / 32)^2 blocks,
    // from block blk_off[b] of the head's region, its range limited to the
    // blocks the offsets give it.
    const int kb32 = kw / 32;
    const uint32_t ds_lane = (uint32_t)lane * 16u;
    const int nb32s = VARLEN ? (N + 31) / 32 : p.nb32;
    size_t ds_seq = 0;
    uint32_t ds_range = p.ds_head;
    if constexpr (VARLEN && STORE_DS) {
      const int o0 = p.blk_off[b], o1 = p.blk_off[b + 1];
      ds_seq = (size_t)o0 * 2048;
      ds_range = (uint32_t)max(o1 - o0, 0) * 2048u;
    }
    auto store_ds = [&](int u, u32x4 w) {
      if constexpr (STORE_DS) {
        const size_t hidx = (VARLEN ? 0 : (size_t)b * p.Hq) + hq0 + cur_g;
        const rsrc_t r = make_rsrc_uniform(p.ds + hidx * p.ds_head + ds_seq, ds_range);
        const uint64_t boff = ((uint64_t)cur_qs * (uint64_t)nb32s + (uint64_t)kb32) * 2048u;
        const bool ok = cur_qs < nb32s && kb32 < nb32s && (!CAUSAL || kb32 <= cur_qs) &&
                        boff + 2048u <= (uint64_t)ds_range;
        const uint32_t off = ok ? (uint32_t)boff : 0xFFFFF000u;
        // Non-temporal (NT): dS is read once, by the dQ pass, so the caches
        // keep K, V and the step tiles instead, and the dQ pass does not first
        // write back lines left dirty here.
        __builtin_amdgcn_raw_buffer_store_b128(w, r, off + ds_lane + 1024u * u, 0, kCachePolicyNT);
      }
    };

    f32x16 sA, dA, sB, dB;
    if (nsteps > 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sA[r] = 0.f;
        dA[r] = 0.f;
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        sA = mfma32(as_bf16x8(*(const u32x4*)(st0 + a_off[t])), kB[t], sA);
        dA = mfma32(as_bf16x8(*(const u32x4*)(st0 + TB + a_off[t])), vB[t], dA);
      }
    }

    // PREF: carried from one iteration to the next, the row constants of the
    // step being finished and the first PD operand pairs of S, dP of the next
    // one, read before the barrier (after this wave's P, dS writes are
    // complete), so the first products of an iteration start right after it.
    constexpr int PD = 2;  // operand read distance, in MFMA pairs
    bf16x8 opA[T], opB[T];
    // Row constants of register r (query 8(r/4) + 4h + r%4 of the step):
    // LSE log2 e as lc[r/4][r%4]; Delta held once per 16-lane row, lane j of
    // the row holding register j's value, and broadcast by DPP where it is
    // used (one LDS read instead of four).
    f32x4 lc[4];
    float dcl;
    const int dc_pos = 8 * ((lane & 15) >> 2) + 4 * h + (lane & 3);
    auto prefetch = [&](const char* rows, const char* ops) __attribute__((always_inline)) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        lc[r4] = *(const f32x4*)((const float*)(rows + 2 * TB) + 8 * r4 + 4 * h);
      dcl = *((const float*)(rows + 2 * TB + 256) + dc_pos);
#pragma unroll
      for (int c = 0; c < PD; ++c) {
        opA[c] = as_bf16x8(*(const u32x4*)(ops + a_off[c]));
        opB[c] = as_bf16x8(*(const u32x4*)(ops + TB + a_off[c]));
      }
    };
    if (PREF && nsteps > 0) prefetch(st0, st1);

    // Iteration i: S(i+1), dP(i+1) from stage `nxt`; P(i), dS(i) from sv, dv
    // with step i's LSE and Delta (stage `cur`); P, dS to `pbw`.  PREF: the
    // row constants and first operands were read before the barrier, and the
    // reads for iteration i+1 (stages nxt and `nn`, step i+2, complete since
    // barrier i) close the iteration; that barrier waits for nothing (this
    // wave's LDS writes were waited for, and no copy after it overwrites the
    // stages still being read).
    auto body = [&](int i, const char* cur, const char* nxt, const char* nn, char* pbw, f32x16& sv,
                    f32x16& dv, f32x16& sn, f32x16& dn) __attribute__((always_inline)) {
      if constexpr (PREF)
        plain_barrier();
      else
        lds_barrier();
      if (i >= nsteps) return;
      const int q0 = cur_qs * QS;
      pin(sv);
      pin(dv);
      // Causal mask near the diagonal (S = -inf where key > query) and
      // padding keys (key >= N).  Register r holds query q0 + 8(r/4) + 4h + r%4.
      if ((CAUSAL && (q0 < kw + 31)) || (kw + 32 > N)) {
        keep_branch();
        const int lim = (key >= N) ? 1 << 30 : (CAUSAL ? key - q0 - 4 * h : -1);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + (r & 3) < lim) sv[r] = -__builtin_inff();
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sn[r] = 0.f;
        dn[r] = 0.f;
      }
      auto fetch = [&](int c) {
        if (c < T) {
          opA[c] = as_bf16x8(*(const u32x4*)(nxt + a_off[c]));
          opB[c] = as_bf16x8(*(const u32x4*)(nxt + TB + a_off[c]));
        }
      };
      if constexpr (!PREF) prefetch(cur, nxt);
      char* pw = pbw + kwave * 4096 + lane * 16;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < T; ++j) {
        fetch(j + PD);
        sn = mfma32(opA[j], kB[j], sn);
        dn = mfma32(opB[j], vB[j], dn);
#pragma unroll
        for (int r = EPJ * j; r < EPJ * (j + 1); ++r) {
          const float pv = exp2_hw(__builtin_fmaf(sv[r], p.c, -lc[r >> 2][r & 3]));
          sv[r] = pv;
          dv[r] = pv * (dv[r] - row_bcast(dcl, r));
          if ((r & 7) == 7) {
            const int u = r >> 3;
            u32x4 w1, w2;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              w1[m] = pack_bf16x2(sv[8 * u + 2 * m], sv[8 * u + 2 * m + 1]);
              w2[m] = pack_bf16x2(dv[8 * u + 2 * m], dv[8 * u + 2 * m + 1]);
            }
            *(u32x4*)(pw + u * 1024) = w1;
            *(u32x4*)(pw + (2 + u) * 1024) = w2;
            store_ds(u, w2);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (--cur_qs < qs_first) {
        cur_qs = nqs - 1;
        ++cur_g;
      }
      if constexpr (PREF) {
        __builtin_amdgcn_sched_barrier(0);
        wait_lgkmcnt0();  // this wave's P, dS writes (and every read) complete
        // (No read is left in flight after the last step.)
        if (i + 1 < nsteps) prefetch(nxt, nn);
      }
    };
    // Stages rotate with period 6, P/dS slots and S/dP register sets with 2.
    // Groups of 6 iterations run whole (iterations past nsteps only meet the
    // barrier): conditional exits between bodies make the register allocator
    // copy the accumulators.
    for (int i = 0; i <= nsteps && nsteps > 0; i += 6) {
      body(i, st0, st1, st2, pb0, sA, dA, sB, dB);
      body(i + 1, st1, st2, st3, pb1, sB, dB, sA, dA);
      body(i + 2, st2, st3, st4, pb0, sA, dA, sB, dB);
      body(i + 3, st3, st4, st5, pb1, sB, dB, sA, dA);
      body(i + 4, st4, st5, st0, pb0, sA, dA, sB, dB);
      body(i + 5, st5, st0, st1, pb1, sB, dB, sA, dA);
    }
  } else {
    // ======================= gradient waves =======================
    // Gradient wave g computes one product over all 128 keys: waves 4, 5 dV
    // += P^T dO, waves 6, 7 dK += dS^T Q, each for ND / 2 of the 32-wide d
    // blocks (d-blocks db0 .. db0 + ND/2 - 1, db0 = (g & 1) ND / 2).  Per
    // 16-query k-step the wave reads the four key blocks' A operands (plain
    // 16-byte reads of the score waves' slots) and, by transposing reads of
    // the step tile, one B operand per d-block, each A read feeding ND / 2
    // products and each B read four.  Accumulator [e][j] covers keys
    // k0 + 32 j + 8(r/4) + 4h + r%4 of register r, d = 32 (db0 + e) + n.
    constexpr int NDW = ND / 2;
    const bool gk = kwave >= 2;  // dK (dS^T Q) rather than dV (P^T dO)
    const int db0 = (kwave & 1) * NDW;
    f32x16 acc[NDW][4];
#pragma unroll
    for (int e = 0; e < NDW; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[e][j][r] = 0.f;
    // Transposing B-operand reads of dO / Q (queries 16 u + 8 rd + 4 h + 0..3
    // of column d = 32 db + n): lane j of 16-lane group gq points at row
    // 8 rd + 4 h + j/4 and d = 32 db + 16 (gq & 1) + 4 (j & 3).
    const int tj = lane & 15, gq = lane >> 4;
    uint32_t tr_off[NDW][2];
#pragma unroll
    for (int e = 0; e < NDW; ++e)
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) {
        const int row = 8 * rd + 4 * h + (tj >> 2);
        const int c = 4 * (db0 + e) + 2 * (gq & 1) + ((tj & 3) >> 1);
        tr_off[e][rd] = (uint32_t)(row * RB + ((c ^ tile_swz<D>(row)) * 16) + (tj & 1) * 8);
      }
    const int tile_off = gk ? 0 : TB;      // Q or dO half of the step tile
    const int slot_off = gk ? 2048 : 0;    // dS or P half of each score wave's slot
    // Iteration i: the product of step i-1 (tile `prv`, P and dS in `pbr`).
    auto body = [&](int i, const char* prv, const char* pbr, char* ld) __attribute__((always_inline)) {
      wait_step(i);
      lds_barrier();
      if (i + 4 < nsteps) issue_next(ld);
      if (i == 0 || i > nsteps) return;
      const char* pr = pbr + slot_off + lane * 16;
      const char* tile = prv + tile_off;
      constexpr int NB = 2 * 4;  // (u, key block j), j fastest
      // Operands are read PD key blocks ahead of their products (3 measured
      // 0.2-0.9% faster than 2).
      constexpr int PD = 3;
      bf16x8 pa[NB], ob[2][NDW];
      auto fetch = [&](int jb) {
        if (jb < NB) {
          const int u = jb / 4, j = jb % 4;
          if (j == 0) {
            const int roff = 16 * u * RB;
#pragma unroll
            for (int e = 0; e < NDW; ++e) {
              const u32x2 lo = lds_read_tr16((const lds_void*)(tile + roff + tr_off[e][0]));
              const u32x2 hi = lds_read_tr16((const lds_void*)(tile + roff + tr_off[e][1]));
              ob[u][e] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
          }
          pa[jb] = as_bf16x8(*(const u32x4*)(pr + j * 4096 + u * 1024));
        }
      };
#pragma unroll
      for (int c = 0; c < PD; ++c) fetch(c);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) {
        const int u = jb / 4, j = jb % 4;
        fetch(jb + PD);
#pragma unroll
        for (int e = 0; e < NDW; ++e) acc[e][j] = mfma32(pa[jb], ob[u][e], acc[e][j]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // Step i-1's tile is in stage (i-1) mod 6, its P and dS in slot (i-1) mod 2;
    // step i+4 is copied into stage (i+4) mod 6.
    for (int i = 0; i <= nsteps && nsteps > 0; i += 6) {
      body(i, st5, pb1, st4);
      body(i + 1, st0, pb0, st5);
      body(i + 2, st1, pb1, st0);
      body(i + 3, st2, pb0, st1);
      body(i + 4, st3, pb1, st2);
      body(i + 5, st4, pb0, st3);
    }
    // dK (scaled) or dV, through a buffer range that starts at the tile's
    // first key and ends at the sequence's last, so stores of padding keys are
    // dropped.  With the query heads cut into parts, each part writes fp32
    // partials that bwd_kv_reduce_kernel sums in part order.
    const float osc = gk ? p.scale : 1.f;
    const uint32_t rows = (uint32_t)min(N - k0, BN);
    if (!VARLEN && p.hsplit > 1) {
      const size_t plane = (size_t)BHkv * N * D;
      const float* po = p.kv_part + (size_t)hs * 2 * plane + (gk ? 0 : plane) + ((size_t)bhk * N + k0) * D;
      const rsrc_t orr = make_rsrc_uniform(po, rows * (uint32_t)(D * 4));
#pragma unroll
      for (int e = 0; e < NDW; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 32 * j + 8 * (r >> 2) + 4 * h + (r & 3);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc[e][j][r] * osc), orr,
                                                  (uint32_t)((row * D + 32 * (db0 + e) + n) * 4), 0, 0);
          }
    } else {
      const rsrc_t orr = make_rsrc_uniform((gk ? dK : dV) + kv_head + (size_t)k0 * D, rows * (uint32_t)RB);
#pragma unroll
      for (int e = 0; e < NDW; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 32 * j + 8 * (r >> 2) + 4 * h + (r & 3);
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(pack_bf16x2(acc[e][j][r] * osc, 0.f) & 0xffffu), orr,
                                                  (uint32_t)((row * D + 32 * (db0 + e) + n) * 2), 0, 0);
          }
    }
  }
}

// ---------------------------------------------------------------------------
// Fixed-order dQ kernel.  Workgroup = (batch, query head, 128 queries), 4
// waves of 32 queries.  K/V tiles of 64 keys are copied straight into LDS
// (double-buffered, one barrier per tile) and walked in ascending order:
//   S^T  = K Q^T,  dP^T = V dO^T      (Q, dO resident as B operands)
//   P^T  = exp2(S^T c - LSE log2 e),  dS^T = P^T o (dP^T - Delta)
//   dQ^T += K^T dS^T                  (K^T by transposing reads of the K tile,
//                                      dS^T straight from the accumulators)
// and dQ = scale * dQ^T is written once, so the sum order is fixed.
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(const uint16_t* __restrict__ Q,
                                                        const uint16_t* __restrict__ K,
                                                        const uint16_t* __restrict__ V,
                                                        const uint16_t* __restrict__ dO,
                                                        uint16_t* __restrict__ dQ, BwdParams p,
                                                        int nqb) {
  constexpr int BM = 128, BN = 64, NW = 4;
  constexpr int RB = D * 2;
  constexpr int KCH = D / 8;
  constexpr int TB = BN * RB;
  constexpr int NLD = TB / 1024 / NW;
  static_assert(NLD >= 1, "tile too small");
  // Two stages of [K, V] tiles as two arrays (so the compiler can tell an
  // in-flight copy into one from reads of the other).
  __shared__ __attribute__((aligned(1024))) char kv0[2 * TB];
  __shared__ __attribute__((aligned(1024))) char kv1[2 * TB];

  // Work item: (batch or sequence, query head, 128-query tile); variable
  // length takes (sequence, tile) pairs from a list sorted largest first.
  const int wg = blockIdx.x;
  int qb, hq, N;
  size_t qrow, kvrow;   // first row of this (sequence, head) in Q/dO/dQ and in K/V
  if constexpr (VARLEN) {
    const int item = wg / p.Hq;
    hq = wg % p.Hq;
    if (item >= *p.n_items) return;
    const int b = p.items[2 * item];
    qb = p.items[2 * item + 1];
    const int s0 = min(max(p.cu[b], 0), p.total);
    N = min(max(p.cu[b + 1] - s0, 0), p.total - s0);
    qrow = (size_t)hq * p.total + s0;
    kvrow = (size_t)(hq / p.G) * p.total + s0;
  } else {
    const int BH = p.B * p.Hq;
    const int bh = wg % BH;
    qb = nqb - 1 - wg / BH;
    const int b = bh / p.Hq;
    hq = bh % p.Hq;
    N = p.N;
    qrow = (size_t)bh * N;
    kvrow = ((size_t)b * (p.Hq / p.G) + hq / p.G) * N;
  }
  const uint32_t head_bytes = (uint32_t)((size_t)N * D * 2);
  const uint16_t* Kh = K + kvrow * D;
  const uint16_t* Vh = V + kvrow * D;

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int n = lane & 31, h = lane >> 5;
  const int q0 = qb * BM;
  const int qw = q0 + wave * 32;
  const int qi = qw + n;

  // Q and dO fragments (B operands; k-step t: d = 16t + 8h .. +8 of query qi).
  const rsrc_t qr = make_rsrc_uniform(Q + qrow * D, head_bytes);
  const rsrc_t dr = make_rsrc_uniform(dO + qrow * D, head_bytes);
  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    qf[t] = as_bf16x8(buf_load16(qr, (uint32_t)(qi * RB + 32 * t + 16 * h)));
    df[t] = as_bf16x8(buf_load16(dr, (uint32_t)(qi * RB + 32 * t + 16 * h)));
  }
  // Row constants of this lane's query (rows past N read as 0; their results
  // are dropped at the store).
  const rsrc_t lr = make_rsrc_uniform(p.lse2 + qrow, (uint32_t)N * 4u);
  const rsrc_t er = make_rsrc_uniform(p.delta + qrow, (uint32_t)N * 4u);
  const float lse2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lr, (uint32_t)qi * 4u, 0, 0));
  const float dlt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(er, (uint32_t)qi * 4u, 0, 0));

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  const int kend = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kend + BN - 1) / BN;

  uint32_t ld_off[NLD];
#pragma unroll
  for (int s = 0; s < NLD; ++s) {
    const int g = (s * NW + wave) * 64 + lane;
    const int row = g / KCH, pc = g % KCH;
    ld_off[s] = (uint32_t)(row * RB + ((pc ^ tile_swz<D>(row)) * 16));
  }
  auto issue_tile = [&](int kt, char* ks) {
    const uint32_t base = (uint32_t)kt * TB;
    const uint32_t left = head_bytes > base ? head_bytes - base : 0u;
    const rsrc_t kr = make_rsrc_uniform((const char*)Kh + base, left);
    const rsrc_t vr = make_rsrc_uniform((const char*)Vh + base, left);
#pragma unroll
    for (int s = 0; s < NLD; ++s) {
      lds_dma16(kr, (lds_void*)(ks + (s * NW + wave) * 1024), ld_off[s]);
      lds_dma16(vr, (lds_void*)(ks + TB + (s * NW + wave) * 1024), ld_off[s]);
    }
  };
  // Row reads (A operands of S^T and dP^T): row n (+32 sb), logical chunk 2t + h.
  uint32_t a_off[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) a_off[t] = (uint32_t)(n * RB + (((2 * t + h) ^ tile_swz<D>(n)) * 16));
  // Transposing reads of K (A operand K^T of dQ^T): in 16-lane group gq, lane j
  // points at key row 8 rd + 4h + j/4 (+ 32 sb + 16 u), d = 32 db + 16 (gq & 1) + 4 (j & 3).
  uint32_t t_off[D / 32][2];
  {
    const int j = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int row = 8 * rd + 4 * h + (j >> 2);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int c = 4 * db + 2 * (gq & 1) + ((j & 3) >> 1);
        t_off[db][rd] = (uint32_t)(row * RB + ((c ^ tile_swz<D>(row)) * 16) + (j & 1) * 8);
      }
    }
  }

  auto tile = [&](int kt, const char* ks, char* next) {
    wait_vmcnt<0>();
    __syncthreads();
    if (kt + 1 < ntiles) issue_tile(kt + 1, next);
    const int k0 = kt * BN;
    if (CAUSAL && k0 > qw + 31) return;
    const char* vs = ks + TB;

    f32x16 st[2], dp[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        st[sb][r] = 0.f;
        dp[sb][r] = 0.f;
      }
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const bf16x8 ka = as_bf16x8(*(const u32x4*)(ks + sb * 32 * RB + a_off[t]));
        const bf16x8 va = as_bf16x8(*(const u32x4*)(vs + sb * 32 * RB + a_off[t]));
        st[sb] = mfma32(ka, qf[t], st[sb]);
        dp[sb] = mfma32(va, df[t], dp[sb]);
      }
    }
    // Register r of half sb holds key k0 + 32 sb + 8 (r/4) + 4 h + r % 4.
    // Causal mask, and padding keys (key >= N, rows read as zero, whose score
    // 0 can exceed every real score).
    const bool need_mask = (CAUSAL && (k0 + BN - 1 > qw)) || (k0 + BN > N);
    const int lim = CAUSAL ? min(qi, N - 1) - k0 - 4 * h : N - 1 - k0 - 4 * h;
    bf16x8 dsb[2][2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = exp2_hw(__builtin_fmaf(st[sb][r], p.c, -lse2));
        if (need_mask && (32 * sb + 8 * (r >> 2) + (r & 3) > lim)) pv = 0.f;
        st[sb][r] = pv * (dp[sb][r] - dlt);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(st[sb][8 * u + 2 * j], st[sb][8 * u + 2 * j + 1]);
        dsb[sb][u] = as_bf16x8(w);
      }
    }
    // dQ^T += K^T dS^T.
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const char* base = ks + (32 * sb + 16 * u) * RB;
          const u32x2 lo = lds_read_tr16((const lds_void*)(base + t_off[db][0]));
          const u32x2 hi = lds_read_tr16((const lds_void*)(base + t_off[db][1]));
          const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
          acc[db] = mfma32(as_bf16x8(a), dsb[sb][u], acc[db]);
        }
  };

  if (ntiles > 0) issue_tile(0, kv0);
  for (int kt = 0; kt < ntiles; kt += 2) {
    tile(kt, kv0, kv1);
    if (kt + 1 < ntiles) tile(kt + 1, kv1, kv0);
  }

  // dQ = scale * dQ^T; register r of block db is d = 32 db + 8 (r/4) + 4 h + r % 4.
  const rsrc_t out = make_rsrc_uniform(dQ + qrow * D, head_bytes);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack_bf16x2(acc[db][4 * g] * p.scale, acc[db][4 * g + 1] * p.scale);
      w[1] = pack_bf16x2(acc[db][4 * g + 2] * p.scale, acc[db][4 * g + 3] * p.scale);
      buf_store8(out, (uint32_t)(qi * RB + (32 * db + 8 * g + 4 * h) * 2), w);
    }
}

// ---------------------------------------------------------------------------
// Stored-dS mode: dQ = scale dS K from the dS^T blocks the main kernel wrote.
// Workgroup = (batch, query head, 128 queries), wave = 32 queries (one block
// row); key tiles of 64 (two blocks) in ascending order, so the sum order is
// fixed.  Per tile: K (shared) and this wave's two dS^T blocks are copied
// into LDS; dQ^T += K^T dS^T with both operands by transposing reads.
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256, 2) void bwd_dq_ds_kernel(const uint16_t* __restrict__ K,
                                                           uint16_t* __restrict__ dQ, BwdParams p,
                                                           int nqb) {
  constexpr int BM = 128, BN = 64, NW = 4;
  constexpr int RB = D * 2;
  constexpr int KCH = D / 8;
  constexpr int TB = BN * RB;
  constexpr int NLD = TB / 1024 / NW;
  constexpr int ND = D / 32;
  static_assert(NLD >= 1, "tile too small");
  __shared__ __attribute__((aligned(1024))) char kbuf0[TB];
  __shared__ __attribute__((aligned(1024))) char kbuf1[TB];
  __shared__ __attribute__((aligned(1024))) char dbuf0[NW * 4096];
  __shared__ __attribute__((aligned(1024))) char dbuf1[NW * 4096];

  // Work item: (batch, query head, 128-query tile), or for packed sequences
  // (sequence, tile) pairs from a list sorted largest first, heads fastest.
  const int wg = blockIdx.x;
  int qb, N, nb32;
  size_t qrow, kvrow;   // first row of this (sequence, head) in dQ and in K
  const char* dsh;      // this (sequence, head)'s block grid
  uint32_t ds_range;
  if constexpr (VARLEN) {
    const int item = wg / p.Hq;
    const int hq = wg % p.Hq;
    if (item >= *p.n_items) return;
    const int b = p.items[2 * item];
    qb = p.items[2 * item + 1];
    const int s0 = min(max(p.cu[b], 0), p.total);
    N = min(max(p.cu[b + 1] - s0, 0), p.total - s0);
    nb32 = (N + 31) / 32;
    qrow = (size_t)hq * p.total + s0;
    kvrow = (size_t)(hq / p.G) * p.total + s0;
    const int o0 = p.blk_off[b], o1 = p.blk_off[b + 1];
    dsh = p.ds + (size_t)hq * p.ds_head + (size_t)o0 * 2048;
    ds_range = (uint32_t)max(o1 - o0, 0) * 2048u;
  } else {
    const int BH = p.B * p.Hq;
    const int bh = wg % BH;
    qb = nqb - 1 - wg / BH;
    const int b = bh / p.Hq, hq = bh % p.Hq;
    N = p.N;
    nb32 = p.nb32;
    qrow = (size_t)bh * N;
    kvrow = ((size_t)b * (p.Hq / p.G) + hq / p.G) * N;
    dsh = p.ds + (size_t)bh * p.ds_head;
    ds_range = p.ds_head;
  }
  const uint32_t head_bytes = (uint32_t)((size_t)N * D * 2);
  const uint16_t* Kh = K + kvrow * D;

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int n = lane & 31, h = lane >> 5;
  const int q0 = qb * BM;
  const int qb32 = qb * 4 + wave;   // this wave's query block

  const int kend = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kend + BN - 1) / BN;

  uint32_t ld_off[NLD];
#pragma unroll
  for (int s = 0; s < NLD; ++s) {
    const int g = (s * NW + wave) * 64 + lane;
    const int row = g / KCH, pc = g % KCH;
    ld_off[s] = (uint32_t)(row * RB + ((pc ^ tile_swz<D>(row)) * 16));
  }
  // A stored block holds key row r's positions 16u + 8h .. +8 as 16-byte
  // chunk 64u + 32h + r.  In LDS that chunk goes to 64u + 32h + (r ^ 4h ^ 8u):
  // the copy moves whole 64-byte groups of four chunks, so each 1 KiB half u
  // (copy s = u) is still one contiguous read, and the transposing reads
  // below, 16 key rows of both h at once, hit 64 distinct banks.
  uint32_t ds_src[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) ds_src[s] = (uint32_t)((64 * s + (lane ^ (4 * (lane >> 5) + 8 * s))) * 16);
  auto issue_tile = [&](int kt, char* ks, char* dsb) {
    const uint32_t base = (uint32_t)kt * TB;
    const uint32_t left = head_bytes > base ? head_bytes - base : 0u;
    const rsrc_t kr = make_rsrc_uniform((const char*)Kh + base, left);
#pragma unroll
    for (int s = 0; s < NLD; ++s) lds_dma16(kr, (lds_void*)(ks + (s * NW + wave) * 1024), ld_off[s]);
    // This wave's blocks (qb32, 2kt) and (qb32, 2kt + 1); a block that was
    // never written (padding, or above the diagonal) reads as zeros.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kb32 = 2 * kt + j;
      // Byte offset in 64 bits: with packed sequences a sequence longer than
      // max_seqlen can index past 2^32 bytes, and only blocks inside the
      // sequence's range are read.
      const uint64_t boff = ((uint64_t)qb32 * (uint64_t)nb32 + (uint64_t)kb32) * 2048u;
      const bool ok = qb32 < nb32 && kb32 < nb32 && (!CAUSAL || kb32 <= qb32) &&
                      boff + 2048u <= (uint64_t)ds_range;
      const uint32_t off = ok ? (uint32_t)boff : 0u;
      const rsrc_t dr = make_rsrc_uniform(dsh + off, ok ? 2048u : 0u);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        lds_dma16_nt(dr, (lds_void*)(dsb + wave * 4096 + j * 2048 + s * 1024), ds_src[s]);
    }
  };

  // Transposing reads.  K^T (A operand, row d = 32 db + n, 8 keys): lane j of
  // 16-lane group gq points at key row 8 rd + 4h + j/4 (+ 16 t), d = 32 db +
  // 16 (gq & 1) + 4 (j & 3).  dS^T (B operand, column = block position n, 8
  // keys): key row r = 8 rd + 4h + j/4 (+ 16 t), position 16 (gq & 1) + 4 (j & 3),
  // i.e. half u = gq & 1, h' = (j & 3) / 2, element 4 (j & 1) of LDS chunk
  // 64u + 32h' + (r ^ 4h' ^ 8u) (the 16 t rows add 256 bytes).
  const int j16 = lane & 15, gq = lane >> 4;
  uint32_t t_off[ND][2], s_off[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int row = 8 * rd + 4 * h + (j16 >> 2);
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const int c = 4 * db + 2 * (gq & 1) + ((j16 & 3) >> 1);
      t_off[db][rd] = (uint32_t)(row * RB + ((c ^ tile_swz<D>(row)) * 16) + (j16 & 1) * 8);
    }
    const int su = gq & 1, sh = (j16 & 3) >> 1;
    s_off[rd] = (uint32_t)(wave * 4096 + (64 * su + 32 * sh + (row ^ (4 * sh) ^ (8 * su))) * 16 + (j16 & 1) * 8);
  }

  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  auto tile = [&](int kt, const char* ks, const char* dsb, char* kn, char* dn) {
    wait_vmcnt<0>();
    __syncthreads();  // tile kt in LDS; tile kt-1's buffers free
    if (kt + 1 < ntiles) issue_tile(kt + 1, kn, dn);
    // k-step t covers keys 16t .. 16t + 15 of the tile (block t / 2, rows
    // 16 (t & 1) ..); db fastest so consecutive MFMAs use different
    // accumulators.
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const char* sb = dsb + (t >> 1) * 2048 + (t & 1) * 256;
      const u32x2 slo = lds_read_tr16((const lds_void*)(sb + s_off[0]));
      const u32x2 shi = lds_read_tr16((const lds_void*)(sb + s_off[1]));
      const bf16x8 bs = as_bf16x8(u32x4{slo[0], slo[1], shi[0], shi[1]});
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const char* kb = ks + 16 * t * RB;
        const u32x2 lo = lds_read_tr16((const lds_void*)(kb + t_off[db][0]));
        const u32x2 hi = lds_read_tr16((const lds_void*)(kb + t_off[db][1]));
        acc[db] = mfma32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), bs, acc[db]);
      }
    }
  };

  if (ntiles > 0) issue_tile(0, kbuf0, dbuf0);
  for (int kt = 0; kt < ntiles; kt += 2) {
    tile(kt, kbuf0, dbuf0, kbuf1, dbuf1);
    if (kt + 1 < ntiles) tile(kt + 1, kbuf1, dbuf1, kbuf0, dbuf0);
  }

  // dQ = scale * (dQ^T)^T.  Column n of the accumulator is block position n,
  // i.e. query 16u + 4h' + (i & 3) + 8 (i >> 2) for n = 16u + 8h' + i; row
  // (register r of block db) is d = 32 db + 8 (r/4) + 4 h + r % 4.
  const int pu = n >> 4, ph = (n >> 3) & 1, pi = n & 7;
  const int qi = qb32 * 32 + 16 * pu + 4 * ph + (pi & 3) + 8 * (pi >> 2);
  const rsrc_t out = make_rsrc_uniform(dQ + qrow * D, head_bytes);
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack_bf16x2(acc[db][4 * g] * p.scale, acc[db][4 * g + 1] * p.scale);
      w[1] = pack_bf16x2(acc[db][4 * g + 2] * p.scale, acc[db][4 * g + 3] * p.scale);
      buf_store8(out, (uint32_t)(qi * RB + (32 * db + 8 * g + 4 * h) * 2), w);
    }
}

// ---------------------------------------------------------------------------
// dQ = bf16(scale * dQ_acc), 8 elements per thread.
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(const float* __restrict__ acc,
                                                             uint16_t* __restrict__ dq,
                                                             size_t n8, float scale) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const float4 a = ((const float4*)acc)[2 * i];
  const float4 b = ((const float4*)acc)[2 * i + 1];
  u32x4 w;
  w[0] = pack_bf16x2(a.x * scale, a.y * scale);
  w[1] = pack_bf16x2(a.z * scale, a.w * scale);
  w[2] = pack_bf16x2(b.x * scale, b.y * scale);
  w[3] = pack_bf16x2(b.z * scale, b.w * scale);
  ((u32x4*)dq)[i] = w;
}

template <int D, bool CAUSAL, bool VARLEN = false>
hipError_t launch_atomic_t(const BwdArgs& a, const BwdParams& p, hipStream_t s, unsigned items = 0) {
  const dim3 grid(VARLEN ? items * (unsigned)a.Hkv : (unsigned)(a.B * a.Hkv * p.nkb));
  hipLaunchKernelGGL((bwd_atomic_kernel<D, CAUSAL, VARLEN>), grid, dim3(64 * kBwdWaves), 0, s,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.dout, (uint16_t*)a.dk, (uint16_t*)a.dv, p);
  return hipGetLastError();
}

BwdParams make_params(const BwdArgs& a) {
  const int QS = 4096 / a.D;
  const BwdLayout lay = bwd_layout(a.B, a.Hq, a.Hkv, a.N, a.D, a.deterministic, a.allow_head_split != 0);
  char* ws = (char*)a.workspace;
  BwdParams p;
  p.B = a.B;
  p.Hq = a.Hq;
  p.G = a.Hq / a.Hkv;
  p.N = a.N;
  p.nkb = (a.N + kBwdBN - 1) / kBwdBN;
  p.nqs = (a.N + QS - 1) / QS;
  p.c = a.scale * kLog2e;
  p.scale = a.scale;
  p.dq_acc = a.deterministic == kDqAtomic ? (float*)(ws + lay.dq_acc) : nullptr;
  p.delta = (float*)(ws + lay.delta);
  p.lse2 = (float*)(ws + lay.lse2);
  p.nb32 = (a.N + 31) / 32;
  p.ds_head = (uint32_t)ds_head_bytes(a.N);
  p.ds = a.deterministic == kDqStored ? ws + lay.ds : nullptr;
  p.hsplit = lay.hsplit;
  p.kv_part = lay.hsplit > 1 ? (float*)(ws + lay.kv_part) : nullptr;
  p.cu = nullptr;
  p.blk_off = nullptr;
  p.total = 0;
  p.items = nullptr;
  p.n_items = nullptr;
  return p;
}

template <int D>
hipError_t launch_pre_d(const BwdArgs& a, hipStream_t s) {
  const BwdParams p = make_params(a);
  const int rows = a.B * a.Hq * a.N;
  constexpr int RPB = 256 / (D / 8);
  const int blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3(blocks), dim3(256), 0, s, (const uint16_t*)a.o,
                     (const uint16_t*)a.dout, a.lse, p, rows);
  return hipGetLastError();
}

// dK, dV = bf16 of the sum of the parts' fp32 partials, in part order (4
// elements per thread; n4 = B * Hkv * N * D / 4 per tensor).
__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(const float* __restrict__ part,
                                                            uint16_t* __restrict__ dk,
                                                            uint16_t* __restrict__ dv, size_t n4,
                                                            int parts) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 * n4) return;
  const size_t which = i / n4, j = i % n4;
  const float4* src = (const float4*)part + which * n4 + j;
  float4 acc = src[0];
  for (int s = 1; s < parts; ++s) {
    const float4 x = src[(size_t)s * 2 * n4];
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  u32x2 w;
  w[0] = pack_bf16x2(acc.x, acc.y);
  w[1] = pack_bf16x2(acc.z, acc.w);
  ((u32x2*)(which ? dv : dk))[j] = w;
}

// The warp-specialized kernel runs both fixed-order dQ modes, at D = 64 and
// 128; the atomic mode runs bwd_atomic_kernel.
template <int D, bool CAUSAL, int DQM>
hipError_t launch_ws_t(const BwdArgs& a, const BwdParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(a.B * a.Hkv * p.nkb * p.hsplit));
  hipLaunchKernelGGL((bwd_ws_kernel<D, CAUSAL, DQM, false>), grid, dim3(512), 0, s, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout,
                     (uint16_t*)a.dk, (uint16_t*)a.dv, p);
  if (p.hsplit > 1) {
    const size_t n4 = (size_t)a.B * a.Hkv * a.N * D / 4;
    hipLaunchKernelGGL(bwd_kv_reduce_kernel, dim3((unsigned)((2 * n4 + 255) / 256)), dim3(256), 0,
                       s, (const float*)p.kv_part, (uint16_t*)a.dk, (uint16_t*)a.dv, n4, p.hsplit);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_main_d(const BwdArgs& a, hipStream_t s) {
  const BwdParams p = make_params(a);
  switch (a.deterministic) {
    case kDqAtomic:
      return a.causal ? launch_atomic_t<D, true>(a, p, s) : launch_atomic_t<D, false>(a, p, s);
    case kDqStored:
      return a.causal ? launch_ws_t<D, true, kDqStored>(a, p, s) : launch_ws_t<D, false, kDqStored>(a, p, s);
    default:
      return a.causal ? launch_ws_t<D, true, kDqRecompute>(a, p, s)
                      : launch_ws_t<D, false, kDqRecompute>(a, p, s);
  }
}

template <int D>
hipError_t launch_dq_ds_d(const BwdArgs& a, hipStream_t s) {
  const BwdParams p = make_params(a);
  const int nqb = (a.N + 127) / 128;
  const dim3 grid((unsigned)(a.B * a.Hq * nqb));
  if (a.causal)
    hipLaunchKernelGGL((bwd_dq_ds_kernel<D, true, false>), grid, dim3(256), 0, s, (const uint16_t*)a.k,
                       (uint16_t*)a.dq, p, nqb);
  else
    hipLaunchKernelGGL((bwd_dq_ds_kernel<D, false, false>), grid, dim3(256), 0, s, (const uint16_t*)a.k,
                       (uint16_t*)a.dq, p, nqb);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dq_d(const BwdArgs& a, hipStream_t s) {
  const BwdParams p = make_params(a);
  const int nqb = (a.N + 127) / 128;
  const dim3 grid((unsigned)(a.B * a.Hq * nqb));
  if (a.causal)
    hipLaunchKernelGGL((bwd_dq_kernel<D, true, false>), grid, dim3(256), 0, s, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout,
                       (uint16_t*)a.dq, p, nqb);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, false, false>), grid, dim3(256), 0, s, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout,
                       (uint16_t*)a.dq, p, nqb);
  return hipGetLastError();
}

// Stored-dS mode with packed sequences: where each sequence's dS blocks start
// in a head's region.  blk_off[b] = sum over b' < b of ceil(len_b' / 32)^2
// (each sequence's full square grid of 32 x 32 blocks, of which the causal
// part is written), clamped to the region's cap_blocks.  One workgroup: each
// thread sums a run of sequences, a scan over the 1024 partial sums, then each
// thread writes its run.  cu_seqlens entries are clamped into [0, total] as
// in the other kernels.
constexpr int kOffThreads = 1024;
__global__ __launch_bounds__(kOffThreads) void varlen_block_offsets_kernel(const int* __restrict__ cu,
                                                                          int B, int total,
                                                                          int cap_blocks,
                                                                          int* __restrict__ blk_off) {
  __shared__ long long part[kOffThreads];
  const int tid = threadIdx.x;
  const int per = (B + kOffThreads - 1) / kOffThreads;
  const int b0 = min(tid * per, B), b1 = min(b0 + per, B);
  auto blocks = [&](int b) -> long long {
    const int s0 = min(max(cu[b], 0), total);
    const int len = min(max(cu[b + 1] - s0, 0), total - s0);
    const long long nb = (len + 31) / 32;
    return nb * nb;
  };
  long long sum = 0;
  for (int b = b0; b < b1; ++b) sum += blocks(b);
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kOffThreads; off <<= 1) {
    const long long add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  long long run = tid > 0 ? part[tid - 1] : 0;
  for (int b = b0; b < b1; ++b) {
    blk_off[b] = (int)min(run, (long long)cap_blocks);
    run += blocks(b);
  }
  if (tid == kOffThreads - 1) blk_off[B] = (int)min(part[kOffThreads - 1], (long long)cap_blocks);
}

// Variable-length backward (dQ modes 0, 1 and 2).  The BwdArgs describe the
// packed tensors as one batch of total rows (a.B = 1, a.N = total), so the
// preprocess and the atomic-mode convert run over every row unchanged.
template <int D, bool CAUSAL>
hipError_t launch_bwd_varlen_t(const BwdArgs& a_in, const VarlenArgs& v, hipStream_t s) {
  const VarlenBwdLayout vl = bwd_varlen_layout(v.B, a_in.Hq, v.total, D, a_in.deterministic, v.max_seqlen);
  char* ws = (char*)a_in.workspace;
  int* main_n = (int*)(ws + vl.main_list);
  int* main_items = (int*)(ws + vl.main_list + 256);
  int* dq_n = (int*)(ws + vl.dq_list);
  int* dq_items = (int*)(ws + vl.dq_list + 256);
  const unsigned items_max = (unsigned)varlen_item_capacity(v.B, v.total);
  constexpr int QS = 4096 / D;
  const bool stored = a_in.deterministic == kDqStored;
  // The row constants (and, mode 0, the fp32 dQ accumulator) sit where the
  // dense layout of B = 1, N = total puts them; the stored-dS mode takes the
  // recompute mode's rows-only layout and adds its block grids after it.
  BwdArgs a = a_in;
  if (stored) a.deterministic = kDqRecompute;
  hipError_t e = launch_varlen_schedule(v, CAUSAL, 1, QS, kBwdBN, main_n, main_items, s);
  if (e != hipSuccess) return e;
  if (a_in.deterministic != kDqAtomic) {
    e = launch_varlen_schedule(v, CAUSAL, 0, QS, 128, dq_n, dq_items, s);
    if (e != hipSuccess) return e;
  }
  int* blk_off = (int*)(ws + vl.blk_off);
  if (stored) {
    hipLaunchKernelGGL(varlen_block_offsets_kernel, dim3(1), dim3(kOffThreads), 0, s, v.cu, v.B, v.total,
                       vl.cap_blocks, blk_off);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  e = launch_pre_d<D>(a, s);
  if (e != hipSuccess) return e;
  BwdParams p = make_params(a);
  p.cu = v.cu;
  p.total = v.total;
  p.hsplit = 1;
  p.kv_part = nullptr;
  p.items = main_items;
  p.n_items = main_n;
  if (stored) {
    p.ds = ws + vl.ds;
    p.ds_head = (uint32_t)vl.ds_head;
    p.blk_off = blk_off;
  }
  if (a.deterministic == kDqAtomic) {
    e = launch_atomic_t<D, CAUSAL, true>(a, p, s, items_max);
  } else if (stored) {
    // The warp-specialized kernel over the (sequence, key tile) list, storing dS.
    hipLaunchKernelGGL((bwd_ws_kernel<D, CAUSAL, kDqStored, true>), dim3(items_max * (unsigned)a.Hkv),
                       dim3(512), 0, s, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (const uint16_t*)a.dout, (uint16_t*)a.dk,
                       (uint16_t*)a.dv, p);
    e = hipGetLastError();
  } else {
    // The warp-specialized kernel over the (sequence, key tile) list.
    hipLaunchKernelGGL((bwd_ws_kernel<D, CAUSAL, kDqRecompute, true>), dim3(items_max * (unsigned)a.Hkv),
                       dim3(512), 0, s, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (const uint16_t*)a.dout, (uint16_t*)a.dk,
                       (uint16_t*)a.dv, p);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  if (a.deterministic == kDqAtomic) {
    const size_t n8 = (size_t)a.Hq * v.total * D / 8;
    hipLaunchKernelGGL(bwd_dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                       (const float*)p.dq_acc, (uint16_t*)a.dq, n8, a.scale);
    return hipGetLastError();
  }
  p.items = dq_items;
  p.n_items = dq_n;
  if (stored)
    hipLaunchKernelGGL((bwd_dq_ds_kernel<D, CAUSAL, true>), dim3(items_max * (unsigned)a.Hq), dim3(256), 0,
                       s, (const uint16_t*)a.k, (uint16_t*)a.dq, p, 0);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, true>), dim3(items_max * (unsigned)a.Hq), dim3(256), 0,
                       s, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, (uint16_t*)a.dq, p, 0);
  return hipGetLastError();
}

}  // namespace

size_t varlen_ds_head_bytes(int B, int total, int max_seqlen) {
  // Sum over sequences of ceil(len / 32)^2 <= (sum of ceil(len / 32)) *
  // (largest ceil(len / 32)) <= (ceil(total / 32) + B) * ceil(max_seqlen / 32)
  // when no sequence is longer than max_seqlen.
  const size_t nsum = ((size_t)total + 31) / 32 + (size_t)B;
  const size_t nmax = ((size_t)max_seqlen + 31) / 32;
  return nsum * nmax * 2048;
}

VarlenBwdLayout bwd_varlen_layout(int B, int Hq, int total, int D, int deterministic, int max_seqlen) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  VarlenBwdLayout l;
  const bool stored = deterministic == kDqStored;
  size_t off = bwd_layout(1, Hq, Hq, total, D, stored ? kDqRecompute : deterministic).total;
  l.ds = off;
  l.ds_head = stored ? varlen_ds_head_bytes(B, total, max_seqlen) : 0;
  l.cap_blocks = stored ? (int)(l.ds_head / 2048) : 0;
  off += stored ? up((size_t)Hq * l.ds_head) : 0;
  l.main_list = off;
  off += varlen_workspace_bytes(B, total);
  l.dq_list = off;
  off += varlen_workspace_bytes(B, total);
  l.blk_off = off;
  off += stored ? up((size_t)(B + 1) * 4) : 0;
  l.total = off;
  return l;
}

size_t bwd_varlen_workspace_bytes(int B, int Hq, int total, int D, int deterministic, int max_seqlen) {
  return bwd_varlen_layout(B, Hq, total, D, deterministic, max_seqlen).total;
}

hipError_t launch_bwd_varlen(const BwdArgs& a, const VarlenArgs& v, hipStream_t s) {
  if (a.D == 64)
    return a.causal ? launch_bwd_varlen_t<64, true>(a, v, s) : launch_bwd_varlen_t<64, false>(a, v, s);
  return a.causal ? launch_bwd_varlen_t<128, true>(a, v, s) : launch_bwd_varlen_t<128, false>(a, v, s);
}

size_t ds_head_bytes(int N) {
  const size_t nb = ((size_t)N + 31) / 32;
  return nb * nb * 2048;
}

int bwd_head_split(int B, int Hq, int Hkv, int N, int D, int deterministic) {
  (void)D;
  if (deterministic == kDqAtomic) return 1;
  const int G = Hq / Hkv;
  const long tiles = (long)B * Hkv * ((N + kBwdBN - 1) / kBwdBN);
  int s = 1;
  while (2 * s <= G && G % (2 * s) == 0 && tiles * s < 1024) s *= 2;
  return s;
}

BwdLayout bwd_layout(int B, int Hq, int Hkv, int N, int D, int deterministic, bool allow_head_split) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rows = (size_t)B * Hq * N;
  BwdLayout l;
  l.delta = 0;
  l.lse2 = up(rows * 4);
  l.dq_acc = l.ds = l.lse2 + up(rows * 4);
  size_t extra = 0;
  if (deterministic == kDqAtomic) extra = up(rows * D * 4);
  if (deterministic == kDqStored) extra = up((size_t)B * Hq * ds_head_bytes(N));
  l.kv_part = l.dq_acc + extra;
  l.hsplit = allow_head_split ? bwd_head_split(B, Hq, Hkv, N, D, deterministic) : 1;
  const size_t part = l.hsplit > 1 ? up((size_t)l.hsplit * 2 * B * Hkv * N * D * 4) : 0;
  l.total = l.kv_part + part;
  return l;
}

hipError_t launch_bwd_preprocess(const BwdArgs& a, hipStream_t s) {
  return a.D == 64 ? launch_pre_d<64>(a, s) : launch_pre_d<128>(a, s);
}

hipError_t launch_bwd_main(const BwdArgs& a, hipStream_t s) {
  return a.D == 64 ? launch_main_d<64>(a, s) : launch_main_d<128>(a, s);
}

// ---------------------------------------------------------------------------
// Fixed scratch of the allocation-free backward (fa_bwd_noalloc), for callers
// that cannot allocate device memory.  It holds the per-row Delta and
// LSE * log2(e) of the recompute mode; the preprocess kernel writes every row
// it later reads, so nothing needs clearing between calls.  Each GPU that runs
// the library holds its own copy for the life of the process, and every call
// on that GPU shares it: calls that overlap in time on one GPU race.
static __device__ __align__(256) char scratch[FA_BWD_NOALLOC_SCRATCH_BYTES];

namespace {
// Device address of `scratch` per device, looked up once per device (with
// that device current).  In host code the array's name is only a host-side
// stand-in, so kernels and copies use these addresses, never the name.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

size_t noalloc_scratch_bytes() { return sizeof(scratch); }

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t s) {
  if (a.deterministic == kDqStored) return a.D == 64 ? launch_dq_ds_d<64>(a, s) : launch_dq_ds_d<128>(a, s);
  if (a.deterministic == kDqRecompute) return a.D == 64 ? launch_dq_d<64>(a, s) : launch_dq_d<128>(a, s);
  const BwdParams p = make_params(a);
  const size_t n8 = (size_t)a.B * a.Hq * a.N * a.D / 8;
  hipLaunchKernelGGL(bwd_dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                     (const float*)p.dq_acc, (uint16_t*)a.dq, n8, a.scale);
  return hipGetLastError();
}

}  // namespace fa
