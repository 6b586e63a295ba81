// Exact-attention backward for gfx950 (MI355X): preprocess, main, dQ convert.
//
// The backward recomputes P from Q, K and the forward's LSE instead of
// storing it (hotdry article, kernel-fusion section) and runs five bf16 MFMA
// products per K/V tile and query tile (hotelren summary, sections 4.1-4.2):
//   S  = Q K^T              P  = exp2(S c - LSE log2 e)
//   dP = dO V^T             dS = P o (dP - Delta),  Delta_i = dO_i . O_i
//   dV += P^T dO            dK += dS^T Q            dQ += dS K
// dK and dV of a key tile are owned by one workgroup; dQ is accumulated in an
// fp32 workspace either with atomics or, in deterministic mode, in a fixed
// order (danialwang explainer, sections 05-06).
//
// Layout choices.  S is computed with keys as the MFMA accumulator's column
// (lane) index.  Its accumulator registers are then, unchanged, the A operand
// of P^T dO and dS^T Q (a C-layout tile read as an A operand is its own
// transpose), which is the "compute the transposed form so the result is the
// next product's operand" idea of the danialwang explainer (section 05).  The
// B operands of those two products need 8 queries of one d per lane, so Q and
// dO are also written to LDS transposed, with queries permuted inside each
// group of 16 to match the accumulator's row order.  dQ contracts over keys,
// so dS takes one trip through LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace fa {
namespace {

constexpr int kBwdBN = 128;    // keys per workgroup (32 per wave)
constexpr int kBwdWaves = 4;
constexpr int kMaxSpin = 1 << 18;  // bound on a deterministic-order wait

__device__ __forceinline__ int pos16(int kl) {
  return (kl & 3) | ((kl >> 3) & 1) << 2 | ((kl >> 2) & 1) << 3;
}
// 16-byte chunk swizzle of a transposed Q / dO row holding RCH chunks
// (RCH = QS / 8): distinct chunks for 8 consecutive d (MFMA reads) and
// for d stepping by 8 (staging writes); always < RCH.
template <int RCH>
__device__ __forceinline__ int tswz(int d) {
  if constexpr (RCH >= 8) return (d ^ (d >> 3)) & 7;
  else return ((d >> 1) ^ (d >> 3)) & (RCH - 1);
}

struct BwdParams {
  int B, Hq, G, N;
  int nkb;         // key tiles per head
  int nqs;         // query steps per head
  float c;         // scale * log2(e)
  float scale;
  float* dq_acc;   // fp32 [B][Hq][N][D]
  float* delta;    // fp32 [B][Hq][N]
  int* counters;   // int32 [B][Hq][nqs] (deterministic only)
};

// ---------------------------------------------------------------------------
// Preprocess: Delta_i = sum_d dO[i,d] O[i,d] (fp32), zero the dQ accumulator
// and the order counters.  A row of D bf16 is read by D/8 lanes (16 B each).
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ O,
                                                      const uint16_t* __restrict__ dO,
                                                      BwdParams p, int rows, int ncount) {
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
    float4* z = (float4*)(p.dq_acc + (size_t)row * D + c * 8);
    z[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    z[1] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && c == 0) p.delta[row] = acc;
  const int gid = blockIdx.x * 256 + tid;
  if (p.counters && gid < ncount) p.counters[gid] = 0;
}

// ---------------------------------------------------------------------------
// Main backward kernel.  Workgroup = (batch, K/V head, key tile of 128);
// wave w owns keys 32w..32w+31 of the tile.  Query steps of QS = 4096 / D
// queries (32 for D = 128, 64 for D = 64) are walked from the last one down to
// the first that meets the tile's diagonal, for each of the G query heads.
template <int D, bool CAUSAL, bool DET>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    BwdParams p) {
  constexpr int BN = kBwdBN;
  constexpr int QS = 4096 / D;        // queries per step
  constexpr int NQB = QS / 32;        // 32-query blocks per step
  constexpr int ND = D / 32;          // 32-wide d blocks
  constexpr int KCH = D / 8;          // 16-byte chunks per row
  static_assert(NQB * ND == kBwdWaves, "one dQ output block per wave");

  __shared__ __attribute__((aligned(16))) uint16_t q_s[QS * D];    // row-major, swizzled
  __shared__ __attribute__((aligned(16))) uint16_t do_s[QS * D];
  __shared__ __attribute__((aligned(16))) uint16_t qt_s[D * QS];   // transposed, permuted
  __shared__ __attribute__((aligned(16))) uint16_t dot_s[D * QS];
  __shared__ __attribute__((aligned(16))) uint16_t ds_s[QS * BN];  // dS [query][key], swizzled
  __shared__ __attribute__((aligned(16))) float lse_s[QS];
  __shared__ __attribute__((aligned(16))) float dlt_s[QS];

  const int Hkv = p.Hq / p.G;
  const int wg = blockIdx.x;
  const int bhk = wg % (p.B * Hkv);
  const int kb = wg / (p.B * Hkv);
  const int b = bhk / Hkv, hk = bhk % Hkv;
  const int k0 = kb * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int kw = k0 + 32 * wave;     // this wave's first key
  const int key = kw + n;            // key this lane carries as MFMA column

  const size_t kv_head = ((size_t)b * Hkv + hk) * (size_t)p.N * D;
  const uint16_t* __restrict__ Kh = K + kv_head;
  const uint16_t* __restrict__ Vh = V + kv_head;

  // Resident B operands for S = Q K^T and dP = dO V^T (k = d).
  bf16x8 kB[D / 16], vB[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
    if (key < p.N) {
      a = *(const u32x4*)(Kh + (size_t)key * D + 16 * t + 8 * h);
      c = *(const u32x4*)(Vh + (size_t)key * D + 16 * t + 8 * h);
    }
    kB[t] = as_bf16x8(a);
    vB[t] = as_bf16x8(c);
  }
  // Resident B operand for this wave's dQ block (k = keys of the tile):
  // lane (d, h) holds K[k0 + 16t + 8h + i][d] for i < 8.
  const int dq_qb = wave / ND, dq_db = wave % ND;
  bf16x8 kT[BN / 16];
  {
    const int d = 32 * dq_db + n;
#pragma unroll
    for (int t = 0; t < BN / 16; ++t) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r0 = k0 + 16 * t + 8 * h + 2 * j;
        const uint32_t lo = (r0 < p.N) ? Kh[(size_t)r0 * D + d] : 0u;
        const uint32_t hi = (r0 + 1 < p.N) ? Kh[(size_t)(r0 + 1) * D + d] : 0u;
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

  // Staging roles: threads 0..127 load Q, 128..255 load dO; each owns 4 rows
  // (queries 4g..4g+3 of the step) of one 16-byte d chunk.
  const int st_half = tid >> 7;            // 0: Q, 1: dO
  const int st_t = tid & 127;
  const int st_c = st_t % KCH, st_g = st_t / KCH;
  static_assert((QS / 4) * KCH == 128, "128 staging threads per tensor");

  // First query step that meets this key tile (causal), else 0.
  const int qs_first = CAUSAL ? (k0 / QS) : 0;

  for (int g = 0; g < p.G; ++g) {
    const int hq = hk * p.G + g;
    const size_t q_head = ((size_t)b * p.Hq + hq) * (size_t)p.N;
    const uint16_t* __restrict__ src = (st_half ? dO : Q) + q_head * D;
    const float* __restrict__ lse_h = LSE + q_head;
    const float* __restrict__ dlt_h = p.delta + q_head;
    float* __restrict__ dq_h = p.dq_acc + q_head * D;

    for (int qs = p.nqs - 1; qs >= qs_first; --qs) {
      const int q0 = qs * QS;
      // ---- stage Q / dO (row-major and transposed), LSE*log2e and Delta ----
      u32x4 rows[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int qr = q0 + 4 * st_g + j;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (qr < p.N) v = *(const u32x4*)(src + (size_t)qr * D + st_c * 8);
        rows[j] = v;
      }
      float lv = 0.f;
      if (tid < QS) {
        const int qr = q0 + tid;
        lv = (qr < p.N) ? lse_h[qr] * kLog2e : __builtin_inff();
      } else if (tid >= 128 && tid < 128 + QS) {
        const int qr = q0 + tid - 128;
        lv = (qr < p.N) ? dlt_h[qr] : 0.f;
      }
      __syncthreads();  // previous step finished reading every LDS buffer
      {
        uint16_t* rm = st_half ? do_s : q_s;
        uint16_t* tr = st_half ? dot_s : qt_s;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * st_g + j;
          *(u32x4*)(rm + r * D + ((st_c ^ (r & 7)) * 8)) = rows[j];
        }
        const int pos = 16 * (st_g >> 2) + pos16(4 * (st_g & 3));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = st_c * 8 + e;
          const int w = e >> 1;
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          u32x2 out;
          out[0] = __builtin_amdgcn_perm(rows[1][w], rows[0][w], sel);
          out[1] = __builtin_amdgcn_perm(rows[3][w], rows[2][w], sel);
          const int chunk = (pos >> 3) ^ tswz<QS / 8>(d);
          *(u32x2*)(tr + d * QS + chunk * 8 + (pos & 7)) = out;
        }
        if (tid < QS) lse_s[tid] = lv;
        else if (tid >= 128 && tid < 128 + QS) dlt_s[tid - 128] = lv;
      }
      __syncthreads();

      // ---- per wave: S, dP, P, dS for each 32-query block; dV, dK --------
      const bool need_mask = (CAUSAL && (q0 < kw + 31)) || (kw + 32 > p.N);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[r] = 0.f;
          dp[r] = 0.f;
        }
        const int qr = 32 * qb + n;  // query row this lane feeds (A operand)
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          const int c = (2 * t + h) ^ (qr & 7);
          const bf16x8 qa = as_bf16x8(*(const u32x4*)(q_s + qr * D + c * 8));
          const bf16x8 da = as_bf16x8(*(const u32x4*)(do_s + qr * D + c * 8));
          s = mfma32(qa, kB[t], s);
          dp = mfma32(da, vB[t], dp);
        }
        // Accumulator register r holds query 32qb + 8(r/4) + 4h + r%4, key `key`.
        bf16x8 pa[2], dsa[2];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int ql = 32 * qb + 8 * r4 + 4 * h;
          const f32x4 l4 = *(const f32x4*)(lse_s + ql);
          const f32x4 d4 = *(const f32x4*)(dlt_s + ql);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 4 * r4 + j;
            float pv = exp2_hw(__builtin_fmaf(s[r], p.c, -l4[j]));
            if (need_mask) {
              const int qg = q0 + ql + j;
              const bool dead = key >= p.N || (CAUSAL && key > qg);
              if (dead) pv = 0.f;
            }
            s[r] = pv;
            dp[r] = pv * (dp[r] - d4[j]);
          }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          u32x4 w1, w2;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            w1[j] = pack_bf16x2(s[8 * u + 2 * j], s[8 * u + 2 * j + 1]);
            w2[j] = pack_bf16x2(dp[8 * u + 2 * j], dp[8 * u + 2 * j + 1]);
          }
          pa[u] = as_bf16x8(w1);
          dsa[u] = as_bf16x8(w2);
        }
        // dV += P^T dO, dK += dS^T Q: B operand lane (d, h) reads 8 queries.
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const int d = 32 * db + n;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int chunk = (2 * (2 * qb + u) + h) ^ tswz<QS / 8>(d);
            const bf16x8 ob = as_bf16x8(*(const u32x4*)(dot_s + d * QS + chunk * 8));
            const bf16x8 qbv = as_bf16x8(*(const u32x4*)(qt_s + d * QS + chunk * 8));
            dv_acc[db] = mfma32(pa[u], ob, dv_acc[db]);
            dk_acc[db] = mfma32(dsa[u], qbv, dk_acc[db]);
          }
        }
        // dS -> LDS as [query][key] (bf16), for the dQ product.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = 32 * qb + 8 * (r >> 2) + 4 * h + (r & 3);
          const int kl = 32 * wave + n;
          const int chunk = (kl >> 3) ^ (ql & 7);
          const uint32_t bits = pack_bf16x2(dp[r], 0.f) & 0xffffu;
          ds_s[ql * BN + chunk * 8 + (kl & 7)] = (uint16_t)bits;
        }
      }
      __syncthreads();

      // ---- dQ block (32 queries x 32 d) of this wave: dS (keys) . K ------
      {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        const int qr = 32 * dq_qb + n;
#pragma unroll
        for (int t = 0; t < BN / 16; ++t) {
          const int c = (2 * t + h) ^ (qr & 7);
          const bf16x8 a = as_bf16x8(*(const u32x4*)(ds_s + qr * BN + c * 8));
          acc = mfma32(a, kT[t], acc);
        }
        // acc register r: query 32 dq_qb + 8(r/4) + 4h + r%4, d = 32 dq_db + n.
        const int d = 32 * dq_db + n;
        if (!DET) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qg = q0 + 32 * dq_qb + 8 * (r >> 2) + 4 * h + (r & 3);
            if (qg < p.N) atomicAdd(dq_h + (size_t)qg * D + d, acc[r]);
          }
        } else {
          // Fixed order: key tiles add into a query step in ascending order.
          // Thread 0 waits (bounded) until this tile's turn, the workgroup
          // adds with plain coherent loads/stores, then publishes the turn.
          int* cnt = p.counters + ((size_t)b * p.Hq + hq) * p.nqs + qs;
          __shared__ int s_late;
          if (tid == 0) {
            int spins = 0;
            while (__hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != kb &&
                   spins < kMaxSpin) {
              __builtin_amdgcn_s_sleep(1);
              ++spins;
            }
            s_late = spins >= kMaxSpin;
          }
          __syncthreads();
          const bool late = s_late;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qg = q0 + 32 * dq_qb + 8 * (r >> 2) + 4 * h + (r & 3);
            if (qg < p.N) {
              float* ptr = dq_h + (size_t)qg * D + d;
              if (late) {
                atomicAdd(ptr, acc[r]);
              } else {
                const float old = __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(ptr, old + acc[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              }
            }
          }
          __threadfence();
          __syncthreads();
          if (tid == 0) __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }

  // ---- dK (scaled) and dV of this wave's 32 keys ----------------------------
  // Accumulator register r of d-block db: key kw + 8(r/4) + 4h + r%4, d = 32db + n.
  uint16_t* dKh = dK + kv_head;
  uint16_t* dVh = dV + kv_head;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = kw + 8 * (r >> 2) + 4 * h + (r & 3);
      if (kr < p.N) {
        const size_t off = (size_t)kr * D + 32 * db + n;
        dKh[off] = (uint16_t)(pack_bf16x2(dk_acc[db][r] * p.scale, 0.f) & 0xffffu);
        dVh[off] = (uint16_t)(pack_bf16x2(dv_acc[db][r], 0.f) & 0xffffu);
      }
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

template <int D, bool CAUSAL, bool DET>
hipError_t launch_bwd_t(const BwdArgs& a, const BwdParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(a.B * a.Hkv * p.nkb));
  hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL, DET>), grid, dim3(64 * kBwdWaves), 0, s,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.dout, a.lse, (uint16_t*)a.dk, (uint16_t*)a.dv, p);
  return hipGetLastError();
}

BwdParams make_params(const BwdArgs& a) {
  const int QS = 4096 / a.D;
  const BwdLayout lay = bwd_layout(a.B, a.Hq, a.N, a.D, a.deterministic);
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
  p.dq_acc = (float*)(ws + lay.dq_acc);
  p.delta = (float*)(ws + lay.delta);
  p.counters = a.deterministic ? (int*)(ws + lay.counters) : nullptr;
  return p;
}

template <int D>
hipError_t launch_pre_d(const BwdArgs& a, hipStream_t s) {
  const BwdParams p = make_params(a);
  const int rows = a.B * a.Hq * a.N;
  constexpr int RPB = 256 / (D / 8);
  const int ncount = a.deterministic ? a.B * a.Hq * p.nqs : 0;
  int blocks = (rows + RPB - 1) / RPB;
  blocks = max(blocks, (ncount + 255) / 256);
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3(blocks), dim3(256), 0, s, (const uint16_t*)a.o,
                     (const uint16_t*)a.dout, p, rows, ncount);
  return hipGetLastError();
}

template <int D>
hipError_t launch_main_d(const BwdArgs& a, hipStream_t s) {
  const BwdParams p = make_params(a);
  if (a.causal)
    return a.deterministic ? launch_bwd_t<D, true, true>(a, p, s) : launch_bwd_t<D, true, false>(a, p, s);
  return a.deterministic ? launch_bwd_t<D, false, true>(a, p, s) : launch_bwd_t<D, false, false>(a, p, s);
}

}  // namespace

BwdLayout bwd_layout(int B, int Hq, int N, int D, int deterministic) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int QS = 4096 / D;
  BwdLayout l;
  l.dq_acc = 0;
  l.delta = up((size_t)B * Hq * N * D * 4);
  l.counters = l.delta + up((size_t)B * Hq * N * 4);
  const size_t nqs = (size_t)(N + QS - 1) / QS;
  l.total = l.counters + (deterministic ? up((size_t)B * Hq * nqs * 4) : 0);
  return l;
}

hipError_t launch_bwd_preprocess(const BwdArgs& a, hipStream_t s) {
  return a.D == 64 ? launch_pre_d<64>(a, s) : launch_pre_d<128>(a, s);
}

hipError_t launch_bwd_main(const BwdArgs& a, hipStream_t s) {
  return a.D == 64 ? launch_main_d<64>(a, s) : launch_main_d<128>(a, s);
}

hipError_t launch_bwd_dq_convert(const BwdArgs& a, hipStream_t s) {
  const BwdParams p = make_params(a);
  const size_t n8 = (size_t)a.B * a.Hq * a.N * a.D / 8;
  hipLaunchKernelGGL(bwd_dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                     (const float*)p.dq_acc, (uint16_t*)a.dq, n8, a.scale);
  return hipGetLastError();
}

}  // namespace fa
