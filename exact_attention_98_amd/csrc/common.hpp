// Device helpers shared by the gfx950 attention kernels: MFMA wrappers, bf16
// packing, cross-half reductions, exp2 variants and LDS swizzles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Conditional rescale threshold in log2 units: the accumulator is rescaled
// only when a row max grows by more than log2(256) = 8, so unnormalised
// probabilities stay below 2^8 (hotelren summary, section 3.3).
constexpr float kTau = 8.0f;

// 32x32x16 bf16 MFMA with fp32 accumulate (gfx950).  Operand layout per lane l:
// A holds row m = l % 32 and 8 consecutive k slots of half l / 32; B holds
// column n = l % 32 and the same k slots; the 16 accumulator registers hold
// column n = l % 32 and rows m = 8 * (r / 4) + 4 * (l / 32) + r % 4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

// Two fp32 -> packed bf16x2 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b16) {
  return __builtin_bit_cast(float, b16 << 16);
}

// Combine a value with the same register of lane l ^ 32 (the other half of
// the wave).  This goes through ds_bpermute (__shfl_xor); the gfx950
// v_permlane32_swap builtin is not used because this compiler drops its
// second result (r[0] + r[1] compiles to r[0] + r[0]).
__device__ __forceinline__ float xhalf_max(float v) { return __builtin_fmaxf(v, __shfl_xor(v, 32, 64)); }
__device__ __forceinline__ float xhalf_sum(float v) { return v + __shfl_xor(v, 32, 64); }

// Value of lane R of the caller's 16-lane row, in every lane of that row
// (DPP row_newbcast, CDNA3 and later).  Used as the first operand of a VOP2
// instruction the compiler folds the broadcast into it (v_sub_f32_dpp and
// the like), so it costs no instruction of its own there.  R must be a
// constant; row_bcast() maps an index known after unrolling onto it.
template <int R>
__device__ __forceinline__ float row_bcast_c(float v) {
  static_assert(R >= 0 && R < 16, "lane of a 16-lane row");
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + R, 0xf,
                                                               0xf, true));
}
__device__ __forceinline__ float row_bcast(float v, int r) {
  switch (r) {
    case 0: return row_bcast_c<0>(v);
    case 1: return row_bcast_c<1>(v);
    case 2: return row_bcast_c<2>(v);
    case 3: return row_bcast_c<3>(v);
    case 4: return row_bcast_c<4>(v);
    case 5: return row_bcast_c<5>(v);
    case 6: return row_bcast_c<6>(v);
    case 7: return row_bcast_c<7>(v);
    case 8: return row_bcast_c<8>(v);
    case 9: return row_bcast_c<9>(v);
    case 10: return row_bcast_c<10>(v);
    case 11: return row_bcast_c<11>(v);
    case 12: return row_bcast_c<12>(v);
    case 13: return row_bcast_c<13>(v);
    case 14: return row_bcast_c<14>(v);
    default: return row_bcast_c<15>(v);
  }
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// ---- buffer resources -------------------------------------------------------
// Raw buffer descriptor over [base, base + bytes): loads past `bytes` return
// zero and stores there are dropped, which handles ragged tails without
// branches.  Word 3 0x00020000 is the gfx9-family raw-buffer format.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// Same, for a base and size that are the same in every lane: the values are
// moved to scalar registers so the descriptor needs no per-lane handling.
__device__ __forceinline__ rsrc_t make_rsrc_uniform(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t nb = __builtin_amdgcn_readfirstlane(bytes);
  return make_rsrc((const void*)(((uint64_t)hi << 32) | lo), nb);
}
// Makes a value opaque at this point in program order: it must be computed
// before here and cannot be moved past or re-associated across this point.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(u32x4& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(f32x16& x) { asm volatile("" : "+v"(x)); }
// Keeps the compiler from turning the guarded block into selects that run on
// every path (used for rare, wave-uniform branches).
__device__ __forceinline__ void keep_branch() { asm volatile("" ::: "memory"); }
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
__device__ __forceinline__ void buf_store8(rsrc_t r, uint32_t voff, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, voff, 0, 0);
}
// 16 bytes per lane from global memory straight into LDS
// (buffer_load_dwordx4 ... lds): lane l's bytes land at lds + 16 l, where lds
// is wave-uniform.  Completion is tracked by vmcnt.
typedef __attribute__((address_space(3))) void lds_void;
// Cache-policy operand of the buffer intrinsics: the non-temporal bit (nt
// on gfx950) for data that is written or read exactly once.
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ void lds_dma16(rsrc_t r, lds_void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, 0, 0, 0);
}
// Same, for data read once (non-temporal: not kept in the caches).
__device__ __forceinline__ void lds_dma16_nt(rsrc_t r, lds_void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, 0, 0, kCachePolicyNT);
}
__device__ __forceinline__ void lds_dma4(rsrc_t r, lds_void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 4, voff, 0, 0, 0);
}
__device__ __forceinline__ void buf_atomic_add(rsrc_t r, uint32_t voff, float v) {
  __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v, r, voff, 0, 0);
}
// Wait until at most n vector-memory operations of this wave are in flight.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
}

// Workgroup barrier for loops that keep direct-to-LDS copies in flight across
// it.  __syncthreads' workgroup release fence makes every wave drain vmcnt,
// and the copies count there, so no copy would outlive the barrier it was
// issued before.  This barrier waits only for the wave's own LDS reads and
// writes (lgkmcnt 0).  A wave must already have waited (wait_vmcnt) for the
// copies whose data other waves read after the barrier.  The empty asm
// statements stop the compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait for all of this wave's LDS reads and writes (vmcnt, expcnt not waited for).
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier with no wait at all.  Before it each wave must have waited
// for its own LDS writes (wait_lgkmcnt0) and for the copies whose data other
// waves read after it (wait_vmcnt); LDS reads it leaves in flight must be of
// buffers that nothing writes after it.  The empty asm statements stop the
// compiler from moving memory operations across it.
__device__ __forceinline__ void plain_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- LDS transposing read -------------------------------------------------------
// ds_read_b64_tr_b16: in each group of 16 lanes, lane j supplies the address of
// 4 consecutive bf16 (8 bytes); lane i receives element i % 4 of the chunks
// supplied by lanes i/4 + 4s, s = 0..3.  So if lane j points at row base + j/4,
// column c0 + 4 (j % 4) of a row-major bf16 matrix, lane i receives the column
// c0 + i of rows base .. base + 3.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
__device__ __forceinline__ u32x2 lds_read_tr16(const lds_void* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}

// ---- LDS tile swizzle ------------------------------------------------------------
// Row-major bf16 tiles of D columns keep 16-byte chunk c of row r at chunk
// c ^ tile_swz<D>(r).  gfx950's LDS serves 256 bytes (64 four-byte banks) per
// cycle; with this swizzle both access patterns the kernels use are
// conflict-free:
//   - 16 consecutive rows at one logical chunk (MFMA row operands, ds_read_b128);
//   - 4 consecutive rows (first row a multiple of 4) at 4 consecutive chunks
//     starting at a multiple of 4 (ds_read_b64_tr_b16, 32 lanes).
// D = 128 (256-byte rows): bits 0-1 and 2-3 of r swapped.  D = 64 (128-byte
// rows, two per 256 bytes): a bijection of bits 1-3 of r with bit 1 moved to
// bit 2.  Both depend on r mod 16 only.
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Hardware exp2 (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2 on FMA/ALU units only: x = n + f with n = floor(x), f in [0, 1),
// 2^f ~ 1 + f (c1 + f (c2 + f c3)), and n added to the exponent field
// (hotelren summary, section 3.2; danialwang explainer, 巧招一).  The
// coefficients are a minimax fit of the relative error with p(0) = 1 exactly
// (fit_exp2_poly.py); the fit's bound is 8.6e-5, below bf16's 2^-9.  Inputs
// below -127 give 0 (so a masked -inf gives exactly 0).
constexpr float kExp2C1 = 0.695117295f;
constexpr float kExp2C2 = 0.227643535f;
constexpr float kExp2C3 = 0.0770680308f;
__device__ __forceinline__ float exp2_poly(float x) {
  const float xc = __builtin_fmaxf(x, -127.0f);
  const float n = __builtin_floorf(xc);
  const float f = xc - n;
  float p = __builtin_fmaf(f, kExp2C3, kExp2C2);
  p = __builtin_fmaf(f, p, kExp2C1);
  p = __builtin_fmaf(f, p, 1.0f);
  const int32_t bits = __builtin_bit_cast(int32_t, p) + ((int32_t)n << 23);
  return x < -127.0f ? 0.0f : __builtin_bit_cast(float, bits);
}

// Compile-time bool for generic lambdas (one instantiation per value).
template <bool V>
struct Flag {
  static constexpr bool value = V;
};

}  // namespace fa
