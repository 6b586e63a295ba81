// FP8 (OCP e4m3) forward for gfx950: quantize pass + attention kernel.
//
// The low-precision forward of the hotdry article (the FP8 / "incoherent
// processing" passage of its memory-access section): Q and K are first
// rotated by a fast Walsh-Hadamard transform with random signs (R = diag(s)
// H / sqrt(D), orthogonal, so (Q R)(K R)^T = Q K^T), which spreads outlier
// channels before quantization; then Q, K, V are quantized to e4m3 and both
// products run on the FP8 matrix cores.
//
// Quantize pass (one wave per 64-row tile of one (batch, head), one row per
// lane): rotation in registers (butterflies at distances 1 .. D/2), tile
// amax, e4m3 codes with round-to-nearest-even.  Q and K: codes = e4m3(x 448 /
// amax), dequantization factor amax / 448 per tile.  V: factor 2^e, the
// smallest power of two with amax / 2^e <= 448, so that it can be applied
// exactly by the matrix instruction's block scale; V is stored transposed per
// 64-key tile ([d][64]) with the keys in the order of the attention kernel's
// P registers (position 32h + p holds key 32 (p/16) + 8 ((p%16)/4) + 4h + p%4).
//
// Attention kernel: the pipelined structure of the bf16 forward with
// v_mfma_scale_f32_32x32x64_f8f6f4 for S^T = K Q^T (k = 64 channels per
// instruction) and O^T += V^T P^T (k = the 64 keys of a tile).  The Q and K
// factors scale S in fp32; the V factor is the A-operand block scale.  The
// rescale is the bf16 forward's lazy one (tau = 8, a rescale only when a row's
// maximum grows by more than 2^8).  Each row's P of a tile is stored as
// e4m3(2^k P), k the integer that puts the row's largest value of the tile in
// (2^7, 2^8], with block scale 2^-k (the matrix instruction's per-lane scale
// of the B operand), so every row uses the top of the e4m3 range whatever its
// distance from the reference maximum.  The row sum l adds the fp32 P.
#include "common.hpp"
#include "kernels.hpp"

namespace fa {
namespace {

constexpr int kF8BN = 64, kQT = 64;   // kQT: quantization tile rows
// Waves per workgroup (32 queries each): 8 at D = 128 (two per SIMD, ping-pong
// below), 4 at D = 64 (a tile copy then still has a 1 KiB share per wave).
template <int D>
constexpr int f8_waves() { return D == 128 ? 8 : 4; }
constexpr float kE4M3Max = 448.f;

typedef int v8i __attribute__((ext_vector_type(8)));

// Four fp32 values to e4m3, packed low to high in one dword (round to
// nearest even).
__device__ __forceinline__ uint32_t cvt_fp8x4(float a, float b, float c2, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c2, d, w, true);
  return (uint32_t)w;
}

// Key held at position q (0..63) of a transposed V tile: half h = q / 32,
// slot p = q % 32 of the P^T operand.
__device__ __forceinline__ int vt_key(int q) {
  const int h = q >> 5, p = q & 31;
  return 32 * (p >> 4) + 8 * ((p & 15) >> 2) + 4 * h + (p & 3);
}

// ---------------------------------------------------------------------------
// Quantize pass.  Work items: [Q tiles | K tiles | V tiles], 64 threads each.
template <int D>
__global__ __launch_bounds__(64) void fp8_quant_kernel(const uint16_t* __restrict__ Q,
                                                       const uint16_t* __restrict__ K,
                                                       const uint16_t* __restrict__ V,
                                                       const float* __restrict__ signs,
                                                       Fp8Layout L) {
  __shared__ uint8_t vt[kQT * D];
  int item = blockIdx.x;
  const int nq = L.BHq * L.nt, nk = L.BHkv * L.nt;
  int kind;  // 0 Q, 1 K, 2 V
  if (item < nq) {
    kind = 0;
  } else if (item < nq + nk) {
    kind = 1;
    item -= nq;
  } else {
    kind = 2;
    item -= nq + nk;
  }
  const int head = item / L.nt, tile = item % L.nt;
  const int t = threadIdx.x;
  const int row = tile * kQT + t;
  const uint16_t* src = (kind == 0 ? Q : (kind == 1 ? K : V)) + (size_t)head * L.N * D;
  float x[D];
  if (row < L.N) {
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const u32x4 w = *(const u32x4*)(src + (size_t)row * D + 8 * c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * c + 2 * j] = bf16_bits_to_float(w[j] & 0xffffu);
        x[8 * c + 2 * j + 1] = bf16_bits_to_float(w[j] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d) x[d] = 0.f;
  }
  if (kind < 2 && signs) {
    // x R = (x o s) H / sqrt(D): butterflies (a, b) -> (a + b, a - b).
#pragma unroll
    for (int d = 0; d < D; ++d) x[d] *= signs[d];
#pragma unroll
    for (int hs = 1; hs < D; hs *= 2)
#pragma unroll
      for (int i = 0; i < D; i += 2 * hs)
#pragma unroll
        for (int j = 0; j < hs; ++j) {
          const float a = x[i + j], b = x[i + j + hs];
          x[i + j] = a + b;
          x[i + j + hs] = a - b;
        }
    const float r = 1.f / __builtin_sqrtf((float)D);
#pragma unroll
    for (int d = 0; d < D; ++d) x[d] *= r;
  }
  float amax = 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) amax = fmaxf(amax, fabsf(x[d]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));

  if (kind < 2) {
    const float a = amax > 0.f ? amax : kE4M3Max;
    const float inv = kE4M3Max / a;
    uint8_t* dst = (kind == 0 ? L.q8 : L.k8) + ((size_t)head * L.Np + row) * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float* e = x + 16 * c + 4 * j;
        auto cl = [&](float z) { return fminf(fmaxf(z * inv, -kE4M3Max), kE4M3Max); };
        w[j] = cvt_fp8x4(cl(e[0]), cl(e[1]), cl(e[2]), cl(e[3]));
      }
      *(u32x4*)(dst + 16 * c) = w;
    }
    if (t == 0) (kind == 0 ? L.qs : L.ks)[(size_t)head * L.nt + tile] = a / kE4M3Max;
    return;
  }
  // V: the power of two 2^e with amax <= 448 2^e < 2 amax (exact compares).
  int e = 0;
  if (amax > 0.f) {
    e = ilogbf(amax) - 8;
    while (amax > ldexpf(kE4M3Max, e)) ++e;
    while (amax <= ldexpf(kE4M3Max, e - 1)) --e;
  }
  const float sc = ldexpf(1.f, -e);
  // Codes into LDS as [key][d], then out as [d][64 positions].
#pragma unroll
  for (int c = 0; c < D / 4; ++c) {
    *(uint32_t*)(vt + t * D + 4 * c) = cvt_fp8x4(x[4 * c] * sc, x[4 * c + 1] * sc, x[4 * c + 2] * sc, x[4 * c + 3] * sc);
  }
  __syncthreads();
  uint8_t* dst = L.v8 + ((size_t)head * L.nt + tile) * D * kQT;
  for (int d = t; d < D; d += 64) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t wd = 0;
#pragma unroll
        for (int b8 = 0; b8 < 4; ++b8) wd |= (uint32_t)vt[vt_key(16 * c + 4 * j + b8) * D + d] << (8 * b8);
        w[j] = wd;
      }
      *(u32x4*)(dst + (size_t)d * kQT + 16 * c) = w;
    }
  }
  if (t == 0) L.ve[(size_t)head * L.nt + tile] = e;
}

// ---------------------------------------------------------------------------
// Attention on the quantized tensors.  Workgroup = (b, hq, 128-query tile),
// 4 waves of 32 queries; K and V^T tiles of 64 keys double-buffered in LDS.
// LDS swizzles: a K row of D bytes holds 16-byte chunk c at c ^ fk(row),
// fk(r) = (r >> (D == 128 ? 1 : 2)) & (D/16 - 1); a V^T row of 64 bytes
// holds chunk c at c ^ ((r >> 2) & 3).  Both make the 16 lanes of a
// 16-byte read hit 16 distinct bank groups.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * f8_waves<D>(), 8 / f8_waves<D>()) void fwd_fp8_kernel(
    uint16_t* __restrict__ O, float* __restrict__ LSE, Fp8Layout L, int Hq, int G, int nqb,
    float c) {
  constexpr int NW = f8_waves<D>();
  constexpr bool PING = NW == 8;
  constexpr int BM = 32 * NW, BN = kF8BN;
  constexpr int CH = D / 16;                 // 16-byte chunks per K row
  constexpr int TBK = BN * D;                // bytes of a K tile
  constexpr int TBV = D * BN;                // bytes of a V^T tile
  constexpr int NLD = TBK / 1024 / NW;       // 1 KiB copies per wave per tile
  constexpr int KT = D / 64;                 // k-steps of S^T
  constexpr int ND = D / 32;                 // 32-row d blocks of O^T
  constexpr int SH = D == 128 ? 1 : 2;
  static_assert(NLD >= 1, "tile too small");
  __shared__ __attribute__((aligned(1024))) char kbuf0[TBK];
  __shared__ __attribute__((aligned(1024))) char kbuf1[TBK];
  __shared__ __attribute__((aligned(1024))) char vbuf0[TBV];
  __shared__ __attribute__((aligned(1024))) char vbuf1[TBV];
  // Ping-pong (8 waves): V(kt-1) is still read after barrier kt, so V is
  // four-deep.
  __shared__ __attribute__((aligned(1024))) char vbuf2_[PING ? TBV : 1024];
  __shared__ __attribute__((aligned(1024))) char vbuf3_[PING ? TBV : 1024];
  char* const vbuf2 = PING ? vbuf2_ : vbuf0;
  char* const vbuf3 = PING ? vbuf3_ : vbuf1;  auto fk = [](int r) { return (r >> SH) & (CH - 1); };
  auto fv = [](int r) { return (r >> 2) & 3; };

  const int BH = L.BHq;
  const int wg = blockIdx.x;
  const int bh = wg % BH;
  const int qb = nqb - 1 - wg / BH;
  const int b = bh / Hq, hq = bh % Hq;
  const int Hkv = Hq / G;
  const int bhk = b * Hkv + hq / G;
  const int N = L.N;

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int n = lane & 31, h = lane >> 5;
  const int q0 = qb * BM;
  const int qw = q0 + wave * 32;
  const int qi = qw + n;
  // Lagging half of the ping-pong: waves 4..7 (wave w runs on SIMD w % 4).
  const bool lag = PING && wave >= NW / 2;

  // Q fragments: k-step t holds bytes 64t + 32h .. +32 of row qi (B operand).
  const rsrc_t qr = make_rsrc_uniform(L.q8 + (size_t)bh * L.Np * D, (uint32_t)((size_t)L.Np * D));
  v8i qf[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    const u32x4 lo = buf_load16(qr, (uint32_t)(qi * D + 64 * t + 32 * h));
    const u32x4 hi = buf_load16(qr, (uint32_t)(qi * D + 64 * t + 32 * h + 16));
    qf[t] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  const float dq_q = L.qs[(size_t)bh * L.nt + min(qw / kQT, L.nt - 1)];
  const float* ksc = L.ks + (size_t)bhk * L.nt;
  const int* vex = L.ve + (size_t)bhk * L.nt;
  const float cq = c * dq_q;   // S c = S_codes c dq_q dq_k

  f32x16 oacc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m_ref = -__builtin_inff();
  float l_part = 0.f;

  const int kend = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kend + BN - 1) / BN;

  // Copies: chunk g = (s*NW + wave)*64 + lane of a tile.
  uint32_t kld_off[NLD], vld_off[NLD];
#pragma unroll
  for (int s = 0; s < NLD; ++s) {
    const int g = (s * NW + wave) * 64 + lane;
    kld_off[s] = (uint32_t)((g / CH) * D + (((g % CH) ^ fk(g / CH)) * 16));
    vld_off[s] = (uint32_t)((g / 4) * 64 + (((g % 4) ^ fv(g / 4)) * 16));
  }
  const uint8_t* k8h = L.k8 + (size_t)bhk * L.Np * D;
  const uint8_t* v8h = L.v8 + (size_t)bhk * L.nt * TBV;
  auto issue_k = [&](int kt, char* dst) {
    const rsrc_t r = make_rsrc_uniform(k8h + (size_t)kt * TBK, (uint32_t)TBK);
#pragma unroll
    for (int s = 0; s < NLD; ++s) lds_dma16(r, (lds_void*)(dst + (s * NW + wave) * 1024), kld_off[s]);
  };
  auto issue_v = [&](int kt, char* dst) {
    const rsrc_t r = make_rsrc_uniform(v8h + (size_t)kt * TBV, (uint32_t)TBV);
#pragma unroll
    for (int s = 0; s < NLD; ++s) lds_dma16(r, (lds_void*)(dst + (s * NW + wave) * 1024), vld_off[s]);
  };
  // LDS read offsets.  K (A operand of S^T): row n (+32 sb), logical chunks
  // 4t + 2h + u.  V^T (A operand of O^T): row n (+32 db), chunks 2h + u.
  uint32_t k_off[KT][2], v_off[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
#pragma unroll
    for (int t = 0; t < KT; ++t) k_off[t][u] = (uint32_t)(n * D + (((4 * t + 2 * h + u) ^ fk(n)) * 16));
    v_off[u] = (uint32_t)(n * 64 + (((2 * h + u) ^ fv(n)) * 16));
  }
  auto kread = [&](const char* kb, int sb, int t) {
    const u32x4 lo = *(const u32x4*)(kb + sb * 32 * D + k_off[t][0]);
    const u32x4 hi = *(const u32x4*)(kb + sb * 32 * D + k_off[t][1]);
    return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto vread = [&](const char* vb, int db) {
    const u32x4 lo = *(const u32x4*)(vb + db * 32 * 64 + v_off[0]);
    const u32x4 hi = *(const u32x4*)(vb + db * 32 * 64 + v_off[1]);
    return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto mfma_f8 = [](v8i a, v8i b2, f32x16 acc, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b2, acc, 0, 0, 0, sa, 0, sb);
  };

  auto mask = [&](int kt, f32x16 (&sv)[2]) {
    const int k0 = kt * BN;
    if ((k0 + BN > N) || (CAUSAL && (k0 + BN - 1 > qw))) {
      keep_branch();
      int lim = N - 1 - k0 - 4 * h;
      if (CAUSAL) lim = min(lim, qi - k0 - 4 * h);
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * sb + 8 * (r >> 2) + (r & 3) > lim) sv[sb][r] = -__builtin_inff();
    }
  };
  // Lazy rescale: taken by the whole wave when some row's tile maximum exceeds
  // its reference by more than tau; each row then moves to the larger of the
  // two.
  auto rescale = [&](float m_tile) {
    if (__builtin_amdgcn_ballot_w64(m_tile > m_ref + kTau) != 0) {
      const float m_new = fmaxf(m_ref, m_tile);
      const float alpha = (m_new == -__builtin_inff()) ? 1.f : exp2_hw(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
      m_ref = m_new;
    }
  };

  // Phase A(kt): S^T(kt+1) on the MFMA unit while the VALU forms
  // e4m3(2^k P(kt)) into pb (k in pbk, per row); phase B(kt): O^T += V^T P^T(kt)
  // with the row max of S^T(kt+1).  2^k is folded into the exp2 argument; the
  // tile's sum of 2^k P is scaled by 2^-k into the row sum.
  v8i pb;
  int pbk = 0;
  auto phase_a = [&](int kt, const char* kn, f32x16 (&sv)[2], f32x16 (&sn)[2],
                     float m_tile) __attribute__((always_inline)) {
    rescale(m_tile);
    const float mu = (m_ref == -__builtin_inff()) ? 0.f : m_ref;
    // m_tile - mu <= tau after the rescale, so k >= 0; a row with no key in
    // the tile (m_tile = -inf) gets the cap, and its P are 0 anyway.
    const float kf = fminf(floorf(8.f - (m_tile - mu)), 64.f);
    const float xoff = kf - mu;
    pbk = (int)kf;
    const float ct = cq * ksc[kt];
    float ts = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sn[sb][r] = 0.f;
    // The 2 KT MFMAs of S^T(kt+1) (sub-blocks alternate), each with 16 / KT
    // elements of P(kt): exp2, row sum, e4m3 into the B operand.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 2 * KT; ++j) {
      const int t = j >> 1, sb = j & 1;
      sn[sb] = mfma_f8(kread(kn, sb, t), qf[t], sn[sb], 127, 127);
#pragma unroll
      for (int e = j * (16 / KT); e < (j + 1) * (16 / KT); e += 4) {
        // Slots e .. e+3 = dword e / 4 of the operand: sub-block e / 16,
        // registers e % 16 .. +3.
        const int esb = e >> 4, r = e & 15;
        float pv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          pv[q] = exp2_hw(__builtin_fmaf(sv[esb][r + q], ct, xoff));
          ts += pv[q];
        }
        pb[e >> 2] = (int)cvt_fp8x4(pv[0], pv[1], pv[2], pv[3]);
      }
      pin(ts);
      __builtin_amdgcn_sched_barrier(0);
    }
    l_part = __builtin_fmaf(ts, __builtin_amdgcn_ldexpf(1.f, -pbk), l_part);
    mask(kt + 1, sn);
  };
  auto phase_b = [&](int kt, const char* vc, const f32x16 (&sn)[2],
                     float& m_tile) __attribute__((always_inline)) {
    // V block scale 2^e, P block scale 2^-k (per row: each lane's scale
    // covers the 32 keys of P it holds).
    const int sa = 127 + vex[kt];
    const int sbp = 127 - pbk;
    const float cn = cq * ksc[min(kt + 1, ntiles - 1)];
    float mx = -__builtin_inff();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      oacc[db] = mfma_f8(vread(vc, db), pb, oacc[db], sa, sbp);
#pragma unroll
      for (int e = db * (32 / ND); e < (db + 1) * (32 / ND); ++e) mx = fmaxf(mx, sn[e >> 4][e & 15]);
      pin(mx);
      __builtin_amdgcn_sched_barrier(0);
    }
    m_tile = xhalf_max(mx) * cn;
  };

  f32x16 sA[2], sB[2];
  float m_nxt = -__builtin_inff();  // row maximum of the next tile's S c (log2 units)
  if (ntiles > 0) {
    issue_k(0, kbuf0);
    issue_v(0, vbuf0);
    if (ntiles > 1) issue_k(1, kbuf1);
    wait_vmcnt<0>();
    __syncthreads();
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sA[sb][r] = 0.f;
#pragma unroll
      for (int t = 0; t < KT; ++t) sA[sb] = mfma_f8(kread(kbuf0, sb, t), qf[t], sA[sb], 127, 127);
    }
    mask(0, sA);
    float mx = -__builtin_inff();
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sA[sb][r]);
    m_nxt = xhalf_max(mx) * cq * ksc[0];
  }
  // Tile kt between barrier kt and barrier kt+1: at barrier kt, K(kt+1) and
  // V(kt) are in LDS and the copies of K(kt+2), V(kt+1) are issued.  Leading
  // waves run A(kt), B(kt); with PING the lagging half runs B(kt-1), A(kt),
  // so on each SIMD one wave's exp2 work runs beside the other's products
  // (each wave's own order, and so its results, are unchanged).
  auto run = [&](auto lag_flag) __attribute__((always_inline)) {
    constexpr bool LAG = decltype(lag_flag)::value;
    auto step = [&](int kt, const char* kn, const char* vc, const char* vp, char* kld, char* vld,
                    f32x16 (&sv)[2], f32x16 (&sn)[2]) __attribute__((always_inline)) {
      wait_vmcnt<0>();
      __syncthreads();
      if (kt + 2 < ntiles) issue_k(kt + 2, kld);
      if (kt + 1 < ntiles) issue_v(kt + 1, vld);
      if constexpr (LAG) {
        if (kt > 0) phase_b(kt - 1, vp, sv, m_nxt);
        phase_a(kt, kn, sv, sn, m_nxt);
      } else {
        phase_a(kt, kn, sv, sn, m_nxt);
        phase_b(kt, vc, sn, m_nxt);
      }
    };
    // K(j) in kbuf[j % 2], V(j) in vbuf[j % 4] (vbuf2, vbuf3 alias vbuf0,
    // vbuf1 without PING).
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
    // The lagging waves still owe B(last); its max is not used.
    if constexpr (LAG) {
      if (ntiles > 0) {
        const int r = (ntiles - 1) & 3;
        phase_b(ntiles - 1, r == 0 ? vbuf0 : r == 1 ? vbuf1 : r == 2 ? vbuf2 : vbuf3, sA, m_nxt);
      }
    }
  };
  if (lag)
    run(Flag<true>{});
  else
    run(Flag<false>{});

  // O = O / l (bf16), LSE = (m_ref + log2 l) ln 2.
  const float l_tot = xhalf_sum(l_part);
  const float inv = 1.f / l_tot;
  const uint32_t head_bytes = (uint32_t)((size_t)N * D * 2);
  const rsrc_t orr = make_rsrc_uniform(O + (size_t)bh * N * D, head_bytes);
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
      w[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
      buf_store8(orr, (uint32_t)(qi * D * 2 + (32 * db + 8 * g + 4 * h) * 2), w);
    }
  if (h == 0 && qi < N) LSE[(size_t)bh * N + qi] = (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

template <int D, bool CAUSAL>
hipError_t launch_fp8_t(const FwdArgs& a, const float* signs, const Fp8Layout& L, hipStream_t s) {
  const int items = (L.BHq + 2 * L.BHkv) * L.nt;
  hipLaunchKernelGGL((fp8_quant_kernel<D>), dim3((unsigned)items), dim3(64), 0, s,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, signs, L);
  constexpr int BM = 32 * f8_waves<D>();
  const int nqb = (a.N + BM - 1) / BM;
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3((unsigned)(L.BHq * nqb)),
                     dim3(64 * f8_waves<D>()), 0, s, (uint16_t*)a.o, a.lse, L, a.Hq, a.Hq / a.Hkv, nqb,
                     a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

Fp8Layout fp8_layout(int B, int Hq, int Hkv, int N, int D, void* workspace, size_t* total) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  Fp8Layout L;
  L.N = N;
  L.nt = (N + kQT - 1) / kQT;
  L.Np = L.nt * kQT;
  L.BHq = B * Hq;
  L.BHkv = B * Hkv;
  char* w = (char*)workspace;
  size_t off = 0;
  L.q8 = (uint8_t*)(w + off);
  off += up((size_t)L.BHq * L.Np * D);
  L.k8 = (uint8_t*)(w + off);
  off += up((size_t)L.BHkv * L.Np * D);
  L.v8 = (uint8_t*)(w + off);
  off += up((size_t)L.BHkv * L.Np * D);
  L.qs = (float*)(w + off);
  off += up((size_t)L.BHq * L.nt * 4);
  L.ks = (float*)(w + off);
  off += up((size_t)L.BHkv * L.nt * 4);
  L.ve = (int*)(w + off);
  off += up((size_t)L.BHkv * L.nt * 4);
  if (total) *total = off;
  return L;
}

hipError_t launch_fwd_fp8(const FwdArgs& a, const float* signs, void* workspace, hipStream_t s) {
  const Fp8Layout L = fp8_layout(a.B, a.Hq, a.Hkv, a.N, a.D, workspace, nullptr);
  if (a.D == 64) return a.causal ? launch_fp8_t<64, true>(a, signs, L, s) : launch_fp8_t<64, false>(a, signs, L, s);
  return a.causal ? launch_fp8_t<128, true>(a, signs, L, s) : launch_fp8_t<128, false>(a, signs, L, s);
}

}  // namespace fa
