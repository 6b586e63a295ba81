// Fused exact-attention forward for gfx950 (MI355X).
//
// One workgroup of NW waves owns a tile of 32 NW queries of one (batch, head);
// each wave owns 32 of them, and all share each K/V tile (dense: 8 waves, two
// per SIMD; split-KV: 4, two workgroups per CU).  K/V tiles of 64 keys are copied from HBM
// straight into LDS (buffer_load ... lds, double-buffered, one barrier per
// tile) past the resident Q fragments, and each tile runs
//   S^T = K Q^T          (bf16 MFMA 32x32x16, fp32 accumulate)
//   mask                 (only on tiles that cross the diagonal or the tail)
//   row max              (in-lane over 32 scores, then one cross-half swap)
//   conditional rescale  (only when a row max grows by more than tau = 8)
//   P^T = exp2(S^T c - m_ref), c = scale * log2(e); row sum in fp32
//   O^T += V^T P^T       (P^T used straight from the accumulator registers,
//                         V^T read from row-major V with ds_read_b64_tr_b16)
// and the epilogue applies the one final correction O / l and writes
// LSE = (m_ref + log2 l) ln 2.
//
// Passages: tiled online softmax -- zeeklog FlashAttention-4 article, section
// 4 pseudocode; exp2 with the scale folded in, the cubic exp2 share and the
// conditional rescale with one final correction -- hotelren summary, sections
// 3.2-3.3, and danialwang explainer, section 04; computing the transposed
// product so the result is already the next product's operand -- danialwang
// explainer, section 05 (the detail under "一个体现功力的细节").
//
// Why S^T: the 32x32 MFMA accumulator gives lane l the column l % 32.  With
// queries as columns, each lane holds 16 scores of its own query per 32-key
// block, so the row max and sum are in-lane plus one exchange with lane
// l ^ 32, the per-row rescale factor is a per-lane scalar, and the
// accumulator of S^T is exactly the B operand of O^T += V^T P^T (its rows are
// the contraction index).
//
// LDS layout: K and V tiles are row-major [key][d] with the 16-byte chunk c of
// row r stored at chunk c ^ tile_swz<D>(r), which keeps the row reads of K and
// the transposing reads of V free of bank conflicts.
#include "common.hpp"
#include "kernels.hpp"

namespace fa {
namespace {

constexpr int kFwdWaves = 8;     // dense forward: 8 waves, 256 queries
constexpr int kVarlenWaves = 4;  // variable-length forward: 4 waves, 128 queries (short sequences waste fewer rows)
constexpr int kSplitWaves = 4;   // split-KV: 4 waves, 128 query rows, two workgroups per CU
constexpr int kFwdBM = 32 * kFwdWaves;
constexpr int kVarlenBM = 32 * kVarlenWaves;
constexpr int kSplitBM = 32 * kSplitWaves;
constexpr int kFwdBN = 64;       // keys per K/V tile

// Addressing modes of the forward kernel.
constexpr int kModeDense = 0;   // [B][H][N][D], one workgroup per (b, hq, query tile)
constexpr int kModeVarlen = 1;  // packed sequences, work list sorted longest first
constexpr int kModeSplit = 2;   // query rows of a K/V group, one key range per workgroup

template <int D, bool CAUSAL, int POLYQ, int MODE, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd_kernel(const uint16_t* __restrict__ Q,
                                                     const uint16_t* __restrict__ K,
                                                     const uint16_t* __restrict__ V,
                                                     uint16_t* __restrict__ O,
                                                     float* __restrict__ LSE, FwdParams p) {
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int BM = 32 * NW, BN = kFwdBN;
  constexpr int RB = D * 2;             // bytes per K/V row
  constexpr int KCH = D / 8;            // 16-byte chunks per row
  constexpr int TB = BN * RB;           // bytes per K (or V) tile
  constexpr int NLD = TB / 1024 / NW;  // 1 KiB direct loads per wave per tensor
  static_assert(NLD >= 1, "tile too small");
  // K and V tiles double-buffered separately, each buffer its own array so the
  // compiler can tell an in-flight copy into one from reads of another.  While
  // tile kt is finished (P(kt), O += V(kt) P(kt)), S(kt+1) is computed from
  // K(kt+1); the copies of K(kt+2) and V(kt+1) are in flight.
  __shared__ __attribute__((aligned(1024))) char kbuf0[TB];
  __shared__ __attribute__((aligned(1024))) char kbuf1[TB];
  __shared__ __attribute__((aligned(1024))) char vbuf0[TB];
  __shared__ __attribute__((aligned(1024))) char vbuf1[TB];
  // Ping-pong of the two halves of an 8-wave workgroup (below): two more V
  // buffers.
  constexpr bool PING = NW == 8;
  __shared__ __attribute__((aligned(1024))) char vbuf2_[PING ? TB : 1024];
  __shared__ __attribute__((aligned(1024))) char vbuf3_[PING ? TB : 1024];
  char* const vbuf2 = PING ? vbuf2_ : vbuf0;
  char* const vbuf3 = PING ? vbuf3_ : vbuf1;

  // Work item of this workgroup: (sequence, query head, query tile).
  // Dense grid order: consecutive workgroup ids walk heads first, so with
  // B*Hq a multiple of 8 every tile of a head lands on the same XCD (ids are
  // dealt to the 8 XCDs round-robin) and shares K/V in that XCD's L2; query
  // tiles go from last to first so that, under the causal mask, the longest
  // tiles start first.  Variable length: the ids walk heads first over a list
  // of (sequence, query tile) items sorted by work, largest first (the
  // longest-first scheduling of the danialwang explainer, section 06), and a
  // sequence's rows start at cu_seqlens[b] in every head's [total][D] matrix.
  // Split-KV (decode-shaped queries): the rows of one workgroup are the
  // G * Nq query rows of the G query heads that share K/V head hk (contiguous
  // in [B][Hq][Nq][D]), and the keys are one range of the Nk keys; partial
  // results (O / l and LSE per row) are merged by a second kernel.
  const int wg = blockIdx.x;
  int N, Nkv, qb, hq;   // N: query rows; Nkv: keys this workgroup walks
  int koff = 0;         // index of its first key (split-KV)
  int split = 0;
  const uint16_t *Qh, *Kh, *Vh;
  uint16_t* Oh;
  float* Lh;
  if constexpr (MODE == kModeSplit) {
    int idx = wg;
    const int bhk = idx % p.BH;  // BH = B * Hkv here
    idx /= p.BH;
    qb = idx % p.nqb;            // row block
    split = idx / p.nqb;
    const int b = bhk / (p.Hq / p.G), hk = bhk % (p.Hq / p.G);
    hq = hk * p.G;
    N = p.G * p.Nq;
    koff = split * p.tiles_per_split * kFwdBN;
    Nkv = max(min(p.Nk - koff, p.tiles_per_split * kFwdBN), 0);
    const size_t row0 = ((size_t)b * p.Hq + hq) * p.Nq;
    Qh = Q + row0 * D;
    Oh = O + row0 * D;
    Lh = LSE + row0;
    Kh = K + ((size_t)bhk * p.Nk + koff) * D;
    Vh = V + ((size_t)bhk * p.Nk + koff) * D;
  } else if constexpr (MODE == kModeVarlen) {
    const int item = wg / p.Hq;
    hq = wg % p.Hq;
    if (item >= *p.n_items) return;  // the grid is sized for the worst case
    const int b = p.items[2 * item];
    qb = p.items[2 * item + 1];
    const int s0 = min(max(p.cu[b], 0), p.total);
    N = min(max(p.cu[b + 1] - s0, 0), p.total - s0);
    Nkv = N;
    const int hk = hq / p.G;
    Qh = Q + ((size_t)hq * p.total + s0) * D;
    Oh = O + ((size_t)hq * p.total + s0) * D;
    Kh = K + ((size_t)hk * p.total + s0) * D;
    Vh = V + ((size_t)hk * p.total + s0) * D;
    Lh = LSE + (size_t)hq * p.total + s0;
  } else {
    const int bh = wg % p.BH;
    qb = p.nqb - 1 - wg / p.BH;
    const int b = bh / p.Hq;
    hq = bh % p.Hq;
    const int hk = hq / p.G;
    N = p.N;
    Nkv = N;
    const size_t he = (size_t)N * D;
    Qh = Q + (size_t)bh * he;
    Oh = O + (size_t)bh * he;
    Kh = K + ((size_t)b * (p.Hq / p.G) + hk) * he;
    Vh = V + ((size_t)b * (p.Hq / p.G) + hk) * he;
    Lh = LSE + (size_t)bh * N;
  }
  const uint32_t head_bytes = (uint32_t)((size_t)N * D * 2);  // query rows
  const uint32_t kv_bytes = (uint32_t)((size_t)Nkv * D * 2);

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int n = lane & 31, h = lane >> 5;
  const int q0 = qb * BM;
  const int qw = q0 + wave * 32;   // first query of this wave (uniform)
  const int qi = qw + n;           // this lane's query
  // Lagging half of the ping-pong: waves NW/2 .. NW-1 (wave w runs on SIMD
  // w % 4, so every SIMD holds one wave of each half).
  const bool lag = PING && wave >= NW / 2;

  // Q fragments (B operand of S^T = K Q^T): k-step t covers d in [16t, 16t+16),
  // lane half h holds d = 16t + 8h .. +8 of query qi (rows past N read as 0).
  const rsrc_t qr = make_rsrc_uniform(Qh, head_bytes);
  bf16x8 qf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) qf[t] = as_bf16x8(buf_load16(qr, (uint32_t)(qi * RB + 32 * t + 16 * h)));

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m_ref = -__builtin_inff();
  float l_part = 0.f;  // this lane half's share of the row sum

  // The workgroup walks the tiles up to its last query; each wave computes
  // only those up to its own diagonal (klast) and after that just meets the
  // barriers and takes its share of the copies.  With 256-query workgroups
  // and 64-key tiles, waves 0..5 would otherwise walk 3, 3, 2, 2, 1, 1 tiles
  // that their causal mask clears entirely (about 2.3% of the forward's
  // matrix work, most of it in the short workgroups that run last).  On its
  // last tile a wave still forms S^T(klast+1), unused: leaving those products
  // out through a second instantiation of phase A made the register
  // allocator spill.  Split-KV causal rows see keys up to
  // Nk - Nq + (row mod Nq): no tile-level cut, the mask handles it.
  const int kend = (CAUSAL && MODE != kModeSplit) ? min(N, q0 + BM) : Nkv;
  const int ntiles = (kend + BN - 1) / BN;
  // A wave whose rows all lie past the end (short sequences, ragged tails)
  // computes nothing (klast = -1); its stores fall outside the buffer ranges.
  int klast = (CAUSAL && MODE != kModeSplit) ? min(qw + 31, N - 1) / BN : ntiles - 1;
  if (MODE != kModeSplit && qw >= N) klast = -1;

  // ---- direct HBM -> LDS staging -------------------------------------------
  // Load s of this wave fills LDS chunks g = (s*NW + wave)*64 + lane of the
  // tile: row g / KCH, physical chunk g % KCH, holding logical chunk
  // (g % KCH) ^ f(row).
  uint32_t ld_off[NLD];
#pragma unroll
  for (int s = 0; s < NLD; ++s) {
    const int g = (s * NW + wave) * 64 + lane;
    const int row = g / KCH, pc = g % KCH;
    ld_off[s] = (uint32_t)(row * RB + ((pc ^ tile_swz<D>(row)) * 16));
  }
  auto issue = [&](const uint16_t* src, int kt, char* dst) {
    const uint32_t base = (uint32_t)kt * TB;
    const uint32_t left = kv_bytes > base ? kv_bytes - base : 0u;
    const rsrc_t r = make_rsrc_uniform((const char*)src + base, left);
#pragma unroll
    for (int s = 0; s < NLD; ++s) lds_dma16(r, (lds_void*)(dst + (s * NW + wave) * 1024), ld_off[s]);
  };

  // Per-lane LDS read offsets (buffer, sub-block and step offsets are constants).
  // K (A operand of S^T): row n (+32 sb), logical chunk 2t + h.
  uint32_t k_off[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) k_off[t] = (uint32_t)(n * RB + (((2 * t + h) ^ tile_swz<D>(n)) * 16));
  // V (A operand of O^T = V^T P^T) through transposing reads: in 16-lane group
  // gq = lane / 16, lane j points at row 8 rd + 4 h + j / 4 (+ 32 sb + 16 u)
  // and d = 32 db + 16 (gq & 1) + 4 (j & 3).
  uint32_t v_off[D / 32][2];
  {
    const int j = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int row = 8 * rd + 4 * h + (j >> 2);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int c = 4 * db + 2 * (gq & 1) + ((j & 3) >> 1);
        v_off[db][rd] = (uint32_t)(row * RB + ((c ^ tile_swz<D>(row)) * 16) + (j & 1) * 8);
      }
    }
  }

  constexpr int T = D / 16;
  // LDS read distance: operand fragments are read this many MFMAs (phase A:
  // k-steps) ahead of the instruction that consumes them.
  constexpr int PDA = 1, PDB = 2;
  // Mask keys past the end and, under causal, keys after the query, on the
  // tiles that need it.  Register r of half sb holds key
  // k0 + 32 sb + 8 (r/4) + 4 h + r % 4.
  // Last key each lane's query may see, in this workgroup's key numbering,
  // and the smallest such key over the wave (which decides whether a tile
  // needs the mask).
  int qlast = qi, wave_qlast = qw;
  if constexpr (MODE == kModeSplit) {
    qlast = p.Nk - p.Nq + qi % p.Nq - koff;
    wave_qlast = p.Nk - p.Nq - koff;
  }
  auto mask = [&](int kt, f32x16 (&sv)[2]) {
    const int k0 = kt * BN;
    if ((k0 + BN > Nkv) || (CAUSAL && (k0 + BN - 1 > wave_qlast))) {
      keep_branch();
      int lim = Nkv - 1 - k0 - 4 * h;
      if (CAUSAL) lim = min(lim, qlast - k0 - 4 * h);
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * sb + 8 * (r >> 2) + (r & 3) > lim) sv[sb][r] = -__builtin_inff();
    }
  };
  // Row max of a masked S^T tile (in-lane, then across the lane halves) and
  // the wave's rescale decision: m_new is the candidate new reference.
  auto row_max = [&](const f32x16 (&sv)[2], float& m_new) {
    float mx = __builtin_fmaxf(sv[0][0], sv[0][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(sv[0][r], sv[0][r + 1]));
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(sv[1][r], sv[1][r + 1]));
    mx = xhalf_max(mx);
    m_new = __builtin_fmaxf(m_ref, mx * p.c);
  };
  // Conditional rescale: taken by the whole wave when any of its rows' max
  // grew by more than tau; each row then moves to its own new max.
  auto rescale = [&](float m_new) {
    if (__builtin_amdgcn_ballot_w64(m_new > m_ref + kTau) != 0) {
      const float alpha = (m_new == -__builtin_inff()) ? 1.f : exp2_hw(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
      m_ref = m_new;
    }
  };

  // One tile kt is two phases.  Phase A(kt): sv holds S^T(kt), masked, with
  // m_new its candidate max; P^T(kt) goes to pb and S^T(kt+1) to sn.  Phase
  // B(kt): O^T += V^T P^T(kt) and the candidate max of S^T(kt+1).  Issue order
  // is fixed by hand (sched_barrier fences): the MFMA unit runs one
  // instruction at a time in program order, so each matrix instruction is
  // followed by VALU work that runs under it.
  bf16x8 pb[2][2];
  auto phase_a = [&](int kt, const char* kn, f32x16 (&sv)[2], f32x16 (&sn)[2],
                     float m_new) __attribute__((always_inline)) {
    rescale(m_new);
    const float msub = (m_ref == -__builtin_inff()) ? 0.f : m_ref;

    // Phase A: the 16 MFMAs of S^T(kt+1) (on a stale buffer after the last
    // tile, results unused), each pair with 4 elements of P^T(kt) =
    // exp2(S^T c - m_ref), the row sum and the bf16 packing.
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sn[sb][r] = 0.f;
    // MFMA pair j = k-step t: sub-blocks 0 and 1 alternate, so consecutive
    // MFMAs never accumulate into the same registers.  The K fragments are
    // read PDA k-steps ahead of their MFMAs.
    auto kread = [&](int j, int sb) { return as_bf16x8(*(const u32x4*)(kn + sb * 32 * RB + k_off[j])); };
    // Phase A runs at raised wave priority, so when both waves of a SIMD are
    // ready, the one forming S(kt+1) and the exponentials issues first and
    // the other wave's P V products fill in behind it (dense 8-wave form 1-3%
    // faster at D = 128 and D = 64, variable-length form 2.5%, split-KV equal;
    // priority during phase B instead gave nothing).
    __builtin_amdgcn_s_setprio(1);
    bf16x8 kq[PDA][2];
#pragma unroll
    for (int j = 0; j < PDA; ++j) {
      kq[j][0] = kread(j, 0);
      kq[j][1] = kread(j, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < T; ++j) {
      sn[0] = mfma32(kq[j % PDA][0], qf[j], sn[0]);
      if (j + PDA < T) kq[j % PDA][0] = kread(j + PDA, 0);
      sn[1] = mfma32(kq[j % PDA][1], qf[j], sn[1]);
      if (j + PDA < T) kq[j % PDA][1] = kread(j + PDA, 1);
#pragma unroll
      for (int e = j * (32 / T); e < (j + 1) * (32 / T); ++e) {
        const int esb = e / 16, r = e % 16;
        const float x = __builtin_fmaf(sv[esb][r], p.c, -msub);
        const float ev = ((r & 3) < POLYQ) ? exp2_poly(x) : exp2_hw(x);
        sv[esb][r] = ev;
        l_part += ev;
        if ((r & 7) == 7) {
          const int u = r >> 3;
          u32x4 w;
#pragma unroll
          for (int m = 0; m < 4; ++m) w[m] = pack_bf16x2(sv[esb][8 * u + 2 * m], sv[esb][8 * u + 2 * m + 1]);
          pin(w);
          pb[esb][u] = as_bf16x8(w);
        }
      }
      pin(l_part);
      __builtin_amdgcn_sched_barrier(0);
    }

    __builtin_amdgcn_s_setprio(0);
    mask(kt + 1, sn);
  };

  auto phase_b = [&](const char* vc, const f32x16 (&sn)[2],
                     float& m_new) __attribute__((always_inline)) {
    // Phase B: O^T += V^T P^T(kt), A operand = keys 32 sb + 16 u + 8 rd + 4 h
    // (0..3) of column d = 32 db + n by two transposing reads, PDB MFMAs ahead;
    // the row max of S^T(kt+1) is spread over it.
    constexpr int NB = (D / 32) * 4;
    // MFMA jb: d block db = jb % (D/32) (fastest, so consecutive MFMAs never
    // accumulate into the same registers), key quarter (sb, u) = jb / (D/32).
    auto vread = [&](int jb) {
      const int db = jb % (D / 32), sb = (jb / (D / 32)) >> 1, u = (jb / (D / 32)) & 1;
      const char* base = vc + (32 * sb + 16 * u) * RB;
      const u32x2 lo = lds_read_tr16((const lds_void*)(base + v_off[db][0]));
      const u32x2 hi = lds_read_tr16((const lds_void*)(base + v_off[db][1]));
      return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
    };
    bf16x8 vq[PDB];
#pragma unroll
    for (int jb = 0; jb < PDB; ++jb) vq[jb] = vread(jb);
    float mx = -__builtin_inff();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
      const int db = jb % (D / 32), sb = (jb / (D / 32)) >> 1, u = (jb / (D / 32)) & 1;
      oacc[db] = mfma32(vq[jb % PDB], pb[sb][u], oacc[db]);
      if (jb + PDB < NB) vq[jb % PDB] = vread(jb + PDB);
#pragma unroll
      for (int e = jb * (32 / NB); e < (jb + 1) * (32 / NB); ++e)
        mx = __builtin_fmaxf(mx, sn[e / 16][e % 16]);
      pin(mx);
      __builtin_amdgcn_sched_barrier(0);
    }
    mx = xhalf_max(mx);
    m_new = __builtin_fmaxf(m_ref, mx * p.c);
  };

  f32x16 sA[2], sB[2];
  float m_new = -__builtin_inff();
  if (ntiles > 0) {
    issue(Kh, 0, kbuf0);
    issue(Vh, 0, vbuf0);
    if (ntiles > 1) issue(Kh, 1, kbuf1);
    wait_vmcnt<0>();
    __syncthreads();
    // S^T(0), its mask and row max.
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sA[sb][r] = 0.f;
#pragma unroll
      for (int t = 0; t < T; ++t)
        sA[sb] = mfma32(as_bf16x8(*(const u32x4*)(kbuf0 + sb * 32 * RB + k_off[t])), qf[t], sA[sb]);
    }
    mask(0, sA);
    row_max(sA, m_new);
  }
  // Tile kt between barrier kt and barrier kt+1.  At barrier kt, K(kt+1) and
  // V(kt) are in LDS, and the copies of K(kt+2) and V(kt+1) are issued.  The
  // leading waves run A(kt), B(kt); with PING the lagging half runs B(kt-1),
  // A(kt), so on every SIMD one wave's exp2 work runs beside the other's
  // P V products (their order within each wave is unchanged, so the results
  // are too).  V(kt-1) is then still being read after barrier kt, which is
  // why PING keeps four V buffers.
  auto run = [&](auto lag_flag) __attribute__((always_inline)) {
    constexpr bool LAG = decltype(lag_flag)::value;
    auto step = [&](int kt, const char* kn, const char* vc, const char* vp, char* kld, char* vld,
                    f32x16 (&sv)[2], f32x16 (&sn)[2]) __attribute__((always_inline)) {
      wait_vmcnt<0>();
      __syncthreads();
      if (kt + 2 < ntiles) issue(Kh, kt + 2, kld);
      if (kt + 1 < ntiles) issue(Vh, kt + 1, vld);
      // Split-KV: a wave whose 32 rows all lie past the workgroup's rows
      // (decode groups have fewer rows than waves) only takes its share of
      // the copies.
      if constexpr (MODE == kModeSplit)
        if (qw >= N) return;
      if constexpr (LAG) {
        if (kt > 0 && kt <= klast + 1) phase_b(vp, sv, m_new);
        if (kt <= klast) phase_a(kt, kn, sv, sn, m_new);
      } else {
        if (kt <= klast) {
          phase_a(kt, kn, sv, sn, m_new);
          phase_b(vc, sn, m_new);
        }
      }
    };
    // K(j) lives in kbuf[j % 2] and V(j) in vbuf[j % 4] (vbuf2, vbuf3 alias
    // vbuf0, vbuf1 without PING).
    int kt = 0;
    for (; kt + 4 <= ntiles; kt += 4) {
      step(kt, kbuf1, vbuf0, vbuf3, kbuf0, vbuf1, sA, sB);
      step(kt + 1, kbuf0, vbuf1, vbuf0, kbuf1, vbuf2, sB, sA);
      step(kt + 2, kbuf1, vbuf2, vbuf1, kbuf0, vbuf3, sA, sB);
      step(kt + 3, kbuf0, vbuf3, vbuf2, kbuf1, vbuf0, sB, sA);
    }
    if (kt < ntiles) step(kt, kbuf1, vbuf0, vbuf3, kbuf0, vbuf1, sA, sB);
    if (kt + 1 < ntiles) step(kt + 1, kbuf0, vbuf1, vbuf0, kbuf1, vbuf2, sB, sA);
    if (kt + 2 < ntiles) step(kt + 2, kbuf1, vbuf2, vbuf1, kbuf0, vbuf3, sA, sB);
    // The lagging waves still owe B(last); its max (of a tile past the end)
    // is not used.
    if constexpr (LAG) {
      if (ntiles > 0 && ntiles - 1 <= klast) {
        const int r = (ntiles - 1) & 3;
        phase_b(r == 0 ? vbuf0 : r == 1 ? vbuf1 : r == 2 ? vbuf2 : vbuf3, sA, m_new);
      }
    }
  };
  if (lag)
    run(Flag<true>{});
  else
    run(Flag<false>{});

  // Final correction: O = O / l, LSE = (m_ref + log2 l) ln 2.  Rows past N are
  // dropped by the buffer range.
  const float l_tot = xhalf_sum(l_part);
  if constexpr (MODE == kModeSplit) {
    if (p.splits > 1) {
      // Partial result of this key range, fp32: O / l and LSE; a row that sees
      // no key of the range gives O = 0 and LSE = -inf (weight 0 in the merge).
      const bool none = !(l_tot > 0.f);
      const float pinv = none ? 0.f : 1.f / l_tot;
      const size_t prow = ((size_t)(wg % p.BH) * p.splits + split) * N;
      const rsrc_t por = make_rsrc_uniform(p.o_part + prow * D, (uint32_t)((size_t)N * D * 4));
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = __builtin_bit_cast(uint32_t, oacc[db][4 * g + j] * pinv);
          __builtin_amdgcn_raw_buffer_store_b128(w, por, (uint32_t)((qi * D + 32 * db + 8 * g + 4 * h) * 4), 0, 0);
        }
      if (h == 0 && qi < N)
        p.l_part[prow + qi] = none ? -__builtin_inff() : (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
      return;
    }
  }
  const float inv = 1.f / l_tot;
  const rsrc_t orr = make_rsrc_uniform(Oh, head_bytes);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
      w[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
      buf_store8(orr, (uint32_t)(qi * RB + (32 * db + 8 * g + 4 * h) * 2), w);
    }
  if (h == 0 && qi < N) Lh[qi] = (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

template <int D, bool CAUSAL, int POLYQ>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  FwdParams p;
  p.BH = a.B * a.Hq;
  p.Hq = a.Hq;
  p.G = a.Hq / a.Hkv;
  p.N = a.N;
  p.nqb = (a.N + kFwdBM - 1) / kFwdBM;
  p.c = a.scale * kLog2e;
  const dim3 grid((unsigned)(p.BH * p.nqb));
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, POLYQ, kModeDense, kFwdWaves>), grid, dim3(64 * kFwdWaves), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_c(const FwdArgs& a, hipStream_t s) {
  switch (a.poly_quarters) {
    case 0: return launch_fwd_t<D, CAUSAL, 0>(a, s);
    case 1: return launch_fwd_t<D, CAUSAL, 1>(a, s);
    default: return launch_fwd_t<D, CAUSAL, 2>(a, s);
  }
}

// ---------------------------------------------------------------------------
// Work list of a variable-length batch: every (sequence b, query tile qb), in
// decreasing order of its number of K/V tiles (the work it does), so that the
// longest items start first and no long one is left running alone at the end
// (danialwang explainer, section 06).  One workgroup: a counting sort over the
// cost in LDS.  Equal costs come out in any order; each item writes its own
// rows, so the result does not depend on it.  cu_seqlens entries are clamped
// into [0, total], so no item can address outside the tensors.
constexpr int kSchedThreads = 1024;
constexpr int kSchedMaxCost = 16384 - kSchedThreads - 1;  // histogram + chunk sums <= 64 KiB

// Items are (sequence, tile of `rows` rows).  KIND 0 costs a query tile by
// the 64-key tiles it walks (forward, fixed-order dQ pass); KIND 1 costs a key
// block by the query steps of qstep queries it walks (main backward kernel).
// The list holds at most `cap` items: well-formed offsets give at most
// total / rows + B of them, but overlapping ones (clamping keeps each
// sequence inside [0, total], not apart from the others) can give more, and
// those past the capacity are dropped rather than written past the list.
template <bool CAUSAL, int KIND>
__global__ __launch_bounds__(kSchedThreads) void varlen_schedule_kernel(const int* __restrict__ cu,
                                                                      int B, int total,
                                                                      int max_cost, int qstep,
                                                                      int rows, int cap,
                                                                      int* __restrict__ n_items,
                                                                      int* __restrict__ items) {
  extern __shared__ int sm[];
  int* hist = sm;                    // max_cost + 1 counters, then start offsets
  int* csum = sm + max_cost + 1;     // per-thread chunk sums
  const int tid = threadIdx.x;
  const int ncost = max_cost + 1;
  for (int c = tid; c < ncost; c += kSchedThreads) hist[c] = 0;
  __syncthreads();
  auto seq_len = [&](int b) {
    const int s0 = min(max(cu[b], 0), total);
    return min(max(cu[b + 1] - s0, 0), total - s0);
  };
  auto cost = [&](int len, int qb) {
    if constexpr (KIND == 0) {
      const int kend = CAUSAL ? min(len, (qb + 1) * rows) : len;
      return min((kend + kFwdBN - 1) / kFwdBN, max_cost);
    } else {
      const int nsteps = (len + qstep - 1) / qstep;
      const int first = CAUSAL ? (qb * rows) / qstep : 0;
      return min(max(nsteps - first, 0), max_cost);
    }
  };
  for (int b = tid; b < B; b += kSchedThreads) {
    const int len = seq_len(b);
    for (int qb = 0; qb * rows < len; ++qb) atomicAdd(&hist[cost(len, qb)], 1);
  }
  __syncthreads();
  // Exclusive scan in decreasing cost: slot r = max_cost - c.  Thread t owns
  // slots [t CH, (t+1) CH).
  const int CH = (ncost + kSchedThreads - 1) / kSchedThreads;
  int mine = 0;
  for (int r = tid * CH; r < min((tid + 1) * CH, ncost); ++r) mine += hist[max_cost - r];
  csum[tid] = mine;
  __syncthreads();
  for (int off = 1; off < kSchedThreads; off <<= 1) {  // inclusive scan of the chunk sums
    const int v = tid >= off ? csum[tid - off] : 0;
    __syncthreads();
    csum[tid] += v;
    __syncthreads();
  }
  int run = csum[tid] - mine;
  for (int r = tid * CH; r < min((tid + 1) * CH, ncost); ++r) {
    const int c = max_cost - r;
    const int cnt = hist[c];
    hist[c] = run;
    run += cnt;
  }
  if (tid == kSchedThreads - 1) *n_items = min(csum[tid], cap);
  __syncthreads();
  for (int b = tid; b < B; b += kSchedThreads) {
    const int len = seq_len(b);
    for (int qb = 0; qb * rows < len; ++qb) {
      const int pos = atomicAdd(&hist[cost(len, qb)], 1);
      if (pos < cap) {
        items[2 * pos] = b;
        items[2 * pos + 1] = qb;
      }
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_varlen_t(const FwdArgs& a, const VarlenArgs& v, hipStream_t s) {
  const size_t items_max = (size_t)varlen_item_capacity(v.B, v.total);
  char* ws = (char*)v.workspace;
  int* n_items = (int*)ws;
  int* items = (int*)(ws + 256);
  const hipError_t e = launch_varlen_schedule(v, CAUSAL, 0, 0, kVarlenBM, n_items, items, s);
  if (e != hipSuccess) return e;
  FwdParams p;
  p.BH = 0;
  p.Hq = a.Hq;
  p.G = a.Hq / a.Hkv;
  p.N = 0;
  p.nqb = 0;
  p.c = a.scale * kLog2e;
  p.cu = v.cu;
  p.items = items;
  p.n_items = n_items;
  p.total = v.total;
  const dim3 grid((unsigned)(items_max * a.Hq));
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, 0, kModeVarlen, kVarlenWaves>), grid, dim3(64 * kVarlenWaves), 0, s,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Merge of the split-KV partial results of one query row: with L_s the
// natural-log LSE of key range s and O_s its normalised output,
// LSE = log sum_s exp(L_s) and O = sum_s exp(L_s - LSE) O_s (an exact
// re-weighting; ranges a row cannot see have L_s = -inf and weight 0).  One
// workgroup of 256 threads per row: thread t owns 4 consecutive elements
// (t % (D/4)) of the splits s = t / (D/4) + k SG, so every split's row is read
// by one coalesced sweep and each thread has only splits / SG loads in flight;
// the SG partial sums meet in LDS.
constexpr int kMergeThreads = 256;
template <int D>
__global__ __launch_bounds__(kMergeThreads) void split_merge_kernel(const float* __restrict__ o_part,
                                                                    const float* __restrict__ l_part,
                                                                    uint16_t* __restrict__ O,
                                                                    float* __restrict__ LSE,
                                                                    int rows_grp, int splits) {
  constexpr int E4 = D / 4;                  // float4 columns per row
  constexpr int SG = kMergeThreads / E4;     // split groups
  __shared__ float4 part[SG][E4];
  __shared__ float red[kMergeThreads / 64];
  __shared__ float gsum[SG];
  const int row = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int grp = row / rows_grp, r = row % rows_grp;
  const size_t base = (size_t)grp * splits * rows_grp + r;   // partial row of split 0
  // Largest L_s over the splits (-inf if the row saw no key at all).
  float mx = -__builtin_inff();
  for (int sp = t; sp < splits; sp += kMergeThreads) mx = fmaxf(mx, l_part[base + (size_t)sp * rows_grp]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) red[wv] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int e4 = t % E4, sg = t / E4;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  float sum = 0.f;
#pragma unroll 4
  for (int sp = sg; sp < splits; sp += SG) {
    const size_t pr = base + (size_t)sp * rows_grp;
    const float ls = l_part[pr];
    const float4 o = ((const float4*)(o_part + pr * D))[e4];
    const float wgt = (ls == -__builtin_inff()) ? 0.f : __expf(ls - mx);
    sum += wgt;
    acc.x += wgt * o.x;
    acc.y += wgt * o.y;
    acc.z += wgt * o.z;
    acc.w += wgt * o.w;
  }
  part[sg][e4] = acc;
  // Every thread of a split group saw the same weights: the total weight is
  // the sum of one thread's per group, added in a fixed order.
  if (e4 == 0) gsum[sg] = sum;
  __syncthreads();
  if (sg == 0) {
    float4 a = part[0][e4];
    float tot = gsum[0];
#pragma unroll
    for (int g = 1; g < SG; ++g) {
      const float4 b = part[g][e4];
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
      tot += gsum[g];
    }
    const float inv = 1.f / tot;
    u32x2 w;
    w[0] = pack_bf16x2(a.x * inv, a.y * inv);
    w[1] = pack_bf16x2(a.z * inv, a.w * inv);
    *(u32x2*)(O + (size_t)row * D + 4 * e4) = w;
    if (e4 == 0) LSE[row] = mx + __logf(tot);
  }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_split_t(const FwdArgs& a, const SplitArgs& sa, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int M = G * sa.Nq;
  const int ntiles = (sa.Nk + kFwdBN - 1) / kFwdBN;
  FwdParams p;
  p.BH = a.B * a.Hkv;
  p.Hq = a.Hq;
  p.G = G;
  p.N = 0;
  p.nqb = (M + kSplitBM - 1) / kSplitBM;
  p.c = a.scale * kLog2e;
  p.cu = nullptr;
  p.items = nullptr;
  p.n_items = nullptr;
  p.total = 0;
  p.Nq = sa.Nq;
  p.Nk = sa.Nk;
  p.splits = sa.splits;
  p.tiles_per_split = (ntiles + sa.splits - 1) / sa.splits;
  char* ws = (char*)sa.workspace;
  const size_t rows = (size_t)a.B * a.Hq * sa.Nq;
  p.o_part = (float*)ws;
  p.l_part = (float*)(ws + ((rows * sa.splits * D * 4 + 255) & ~(size_t)255));
  const dim3 grid((unsigned)(p.BH * p.nqb * sa.splits));
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, 0, kModeSplit, kSplitWaves>), grid, dim3(64 * kSplitWaves), 0, s,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, p);
  if (sa.splits > 1)
    hipLaunchKernelGGL((split_merge_kernel<D>), dim3((unsigned)rows), dim3(kMergeThreads), 0, s,
                       (const float*)p.o_part, (const float*)p.l_part, (uint16_t*)a.o, a.lse, M,
                       sa.splits);
  return hipGetLastError();
}

}  // namespace

// Splits for a decode-shaped problem: enough workgroups for two per CU
// (512 on the 256 CUs of an MI355X), without ranges shorter than 4 tiles.
int split_auto(int B, int Hq, int Hkv, int Nq, int Nk) {
  const int M = (Hq / Hkv) * Nq;
  const long base = (long)B * Hkv * ((M + kSplitBM - 1) / kSplitBM);
  const int ntiles = (Nk + kFwdBN - 1) / kFwdBN;
  long want = (512 + base - 1) / base;
  const long cap = (ntiles + 3) / 4;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  return (int)want;
}

int split_max(int Nk) { return (Nk + kFwdBN - 1) / kFwdBN; }

size_t split_workspace_bytes(int B, int Hq, int Nq, int D, int splits) {
  if (splits <= 1) return 0;
  const size_t rows = (size_t)B * Hq * Nq;
  return ((rows * splits * D * 4 + 255) & ~(size_t)255) + ((rows * splits * 4 + 255) & ~(size_t)255);
}

hipError_t launch_fwd_split(const FwdArgs& a, const SplitArgs& sa, hipStream_t s) {
  if (a.D == 64)
    return a.causal ? launch_fwd_split_t<64, true>(a, sa, s) : launch_fwd_split_t<64, false>(a, sa, s);
  return a.causal ? launch_fwd_split_t<128, true>(a, sa, s) : launch_fwd_split_t<128, false>(a, sa, s);
}

hipError_t launch_varlen_schedule(const VarlenArgs& v, int causal, int kind, int qstep, int rows,
                                  int* n_items, int* items, hipStream_t s) {
  // Largest cost: 64-key tiles of the longest sequence (kind 0) or its query
  // steps (kind 1, qstep >= 32 so never more than twice the tiles).
  const int max_cost = kind == 0 ? (v.max_seqlen + kFwdBN - 1) / kFwdBN
                                 : (v.max_seqlen + qstep - 1) / qstep;
  const size_t shm = (size_t)(max_cost + 1 + kSchedThreads) * sizeof(int);
  const int cap = varlen_item_capacity(v.B, v.total);
  if (kind == 0) {
    if (causal)
      hipLaunchKernelGGL((varlen_schedule_kernel<true, 0>), dim3(1), dim3(kSchedThreads), shm, s,
                         v.cu, v.B, v.total, max_cost, qstep, rows, cap, n_items, items);
    else
      hipLaunchKernelGGL((varlen_schedule_kernel<false, 0>), dim3(1), dim3(kSchedThreads), shm, s,
                         v.cu, v.B, v.total, max_cost, qstep, rows, cap, n_items, items);
  } else {
    if (causal)
      hipLaunchKernelGGL((varlen_schedule_kernel<true, 1>), dim3(1), dim3(kSchedThreads), shm, s,
                         v.cu, v.B, v.total, max_cost, qstep, rows, cap, n_items, items);
    else
      hipLaunchKernelGGL((varlen_schedule_kernel<false, 1>), dim3(1), dim3(kSchedThreads), shm, s,
                         v.cu, v.B, v.total, max_cost, qstep, rows, cap, n_items, items);
  }
  return hipGetLastError();
}

// Room for one work list of tiles of at least 128 rows: at most
// sum_b ceil(len_b / 128) <= total / 128 + B items when the sequences do not
// overlap (the schedule kernel drops any beyond that).
int varlen_item_capacity(int B, int total) { return total / 128 + B; }

size_t varlen_workspace_bytes(int B, int total) {
  return 256 + (size_t)varlen_item_capacity(B, total) * 2 * sizeof(int);
}

int varlen_max_seqlen_limit() { return kSchedMaxCost * kFwdBN; }

hipError_t launch_fwd_varlen(const FwdArgs& a, const VarlenArgs& v, hipStream_t s) {
  if (a.D == 64)
    return a.causal ? launch_fwd_varlen_t<64, true>(a, v, s) : launch_fwd_varlen_t<64, false>(a, v, s);
  return a.causal ? launch_fwd_varlen_t<128, true>(a, v, s) : launch_fwd_varlen_t<128, false>(a, v, s);
}

// The forward's FMA-only exp2 on an array, for host-side bit-for-bit checks.
__global__ __launch_bounds__(256) void exp2_poly_eval_kernel(const float* __restrict__ x,
                                                             float* __restrict__ y, int n) {
  const unsigned i = blockIdx.x * 256u + threadIdx.x;  // n <= INT_MAX, so this does not wrap
  if (i < (unsigned)n) y[i] = exp2_poly(x[i]);
}

hipError_t launch_exp2_poly_eval(const float* x, float* y, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(exp2_poly_eval_kernel, dim3((unsigned)(((long long)n + 255) / 256)), dim3(256), 0, s, x, y, n);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  if (a.D == 64) return a.causal ? launch_fwd_c<64, true>(a, s) : launch_fwd_c<64, false>(a, s);
  return a.causal ? launch_fwd_c<128, true>(a, s) : launch_fwd_c<128, false>(a, s);
}

}  // namespace fa
