// Device building blocks for gfx950: dtype decode, 16-byte streaming loads,
// wave64 reductions on DPP, workgroup reductions through LDS, Philox4x32-10,
// uniforms and Gumbel draws.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd.h"

namespace ssd {

constexpr int BLK = SSD_BLOCK;   // vocabulary block (two-level sampler, partials)
constexpr int WG = 256;          // threads per streaming workgroup
constexpr int NWAVE = WG / 64;   // wave64s per streaming workgroup
constexpr int EWG = 256;         // threads per epilogue workgroup (one wave per SIMD)
constexpr int ENW = EWG / 64;
constexpr int MAX_NB = SSD_MAX_V / SSD_BLOCK;
constexpr int CAND_CAP = 256;    // top-F candidate list held in LDS
constexpr int MAX_F = SSD_MAX_F;
constexpr int MAX_K1 = SSD_MAX_K + 1;

constexpr double LOG2E = 1.4426950408889634073599246810019;
constexpr double LN2 = 0.69314718055994530941723212145818;

// ---------------------------------------------------------------------------
// dtype traits: bytes per element, elements per 16-byte chunk, decode
// ---------------------------------------------------------------------------
template <int DT> struct Dt;
template <> struct Dt<SSD_F32> { static constexpr int SZ = 4; static constexpr int VW = 4; };
template <> struct Dt<SSD_BF16> { static constexpr int SZ = 2; static constexpr int VW = 8; };
template <> struct Dt<SSD_F16> { static constexpr int SZ = 2; static constexpr int VW = 8; };

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

template <int DT>
__device__ __forceinline__ void decode16(const uint4 w, float* o) {
  if constexpr (DT == SSD_F32) {
    o[0] = __uint_as_float(w.x); o[1] = __uint_as_float(w.y);
    o[2] = __uint_as_float(w.z); o[3] = __uint_as_float(w.w);
  } else if constexpr (DT == SSD_BF16) {
    o[0] = bf16lo(w.x); o[1] = bf16hi(w.x); o[2] = bf16lo(w.y); o[3] = bf16hi(w.y);
    o[4] = bf16lo(w.z); o[5] = bf16hi(w.z); o[6] = bf16lo(w.w); o[7] = bf16hi(w.w);
  } else {
    o[0] = f16lo(w.x); o[1] = f16hi(w.x); o[2] = f16lo(w.y); o[3] = f16hi(w.y);
    o[4] = f16lo(w.z); o[5] = f16hi(w.z); o[6] = f16lo(w.w); o[7] = f16hi(w.w);
  }
}

// One element (any alignment).
template <int DT>
__device__ __forceinline__ float load_elem(const unsigned char* row, int64_t i) {
  if constexpr (DT == SSD_F32) {
    return reinterpret_cast<const float*>(row)[i];
  } else {
    uint32_t h = reinterpret_cast<const uint16_t*>(row)[i];
    return DT == SSD_BF16 ? __uint_as_float(h << 16)
                          : (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  }
}

// Loads are kept unconditional so that all of a wave's loads are in flight
// together (a load inside a divergent branch gets its own wait): a full
// block takes the plain path; the last, ragged block clamps out-of-range
// addresses to element 0 of the row and replaces those values by -inf.
// The aligned path is taken only when base, row stride and V are 16-byte
// multiples, so a 16-byte chunk is either wholly inside the row or past it.

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// VW consecutive elements from e0 (e0 + VW <= V on the aligned path).  The
// streaming passes read each logit once, so the 16-byte loads carry the
// nontemporal hint (measured ~7% more read bandwidth on gfx950 than plain
// loads over inputs larger than the Infinity Cache).
template <int DT, bool AL>
__device__ __forceinline__ void load_chunk_full(const unsigned char* row, int e0, float* o) {
  constexpr int VW = Dt<DT>::VW;
  if constexpr (AL) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + (size_t)e0 * Dt<DT>::SZ));
    decode16<DT>(make_uint4(t.x, t.y, t.z, t.w), o);
  } else {
#pragma unroll
    for (int e = 0; e < VW; ++e) o[e] = load_elem<DT>(row, e0 + e);
  }
}

// VW consecutive elements from e0; elements at or past V read as -inf.
template <int DT, bool AL>
__device__ __forceinline__ void load_chunk(const unsigned char* row, int V, int e0, float* o) {
  constexpr int VW = Dt<DT>::VW;
  if constexpr (AL) {
    const bool in = e0 < V;
    const uint4 w = *reinterpret_cast<const uint4*>(row + (size_t)(in ? e0 : 0) * Dt<DT>::SZ);
    decode16<DT>(w, o);
#pragma unroll
    for (int e = 0; e < VW; ++e) o[e] = in ? o[e] : -INFINITY;
  } else {
#pragma unroll
    for (int e = 0; e < VW; ++e) {
      const bool in = e0 + e < V;
      const float x = load_elem<DT>(row, in ? e0 + e : 0);
      o[e] = in ? x : -INFINITY;
    }
  }
}

// The 32 elements a lane owns in block beta: chunks lane + 64*i, i < 32/VW.
// Element k = i*VW + e sits at beta*BLK + (i*64 + lane)*VW + e.
// load_block_full: the block lies wholly inside the row (no guards).
// load_block: any block index (past-the-end elements read as -inf).
template <int DT, bool AL>
__device__ __forceinline__ void load_block_full(const unsigned char* row, int beta, int lane, float (&v)[32]) {
  constexpr int VW = Dt<DT>::VW;
  const int base = beta * BLK + lane * VW;
#pragma unroll
  for (int i = 0; i < 32 / VW; ++i) load_chunk_full<DT, AL>(row, base + i * 64 * VW, &v[i * VW]);
}
template <int DT, bool AL>
__device__ __forceinline__ void load_block(const unsigned char* row, int V, int beta, int lane, float (&v)[32]) {
  constexpr int VW = Dt<DT>::VW;
  const int base = beta * BLK + lane * VW;
#pragma unroll
  for (int i = 0; i < 32 / VW; ++i) load_chunk<DT, AL>(row, V, base + i * 64 * VW, &v[i * VW]);
}

// A block as loaded, still packed: 32-bit words per lane (bf16/fp16 keep two
// elements per word on the aligned path, half the registers of decoded
// floats); elements past V hold the bit pattern of -inf.
template <int DT> struct NegInf;
template <> struct NegInf<SSD_F32> { static constexpr uint32_t W = 0xFF800000u; };
template <> struct NegInf<SSD_BF16> { static constexpr uint32_t W = 0xFF80FF80u; static constexpr uint32_t H = 0xFF80u; };
template <> struct NegInf<SSD_F16> { static constexpr uint32_t W = 0xFC00FC00u; static constexpr uint32_t H = 0xFC00u; };

template <int DT, bool AL>
struct RawBlock {
  static constexpr int N = AL ? 8 * Dt<DT>::SZ : 32;
  uint32_t w[N];
};

// NT: full blocks are read with the nontemporal hint (the default: each logit
// is read once), or with ordinary loads for rows a later kernel may re-read.
template <int DT, bool AL, bool FULL, bool NT = true>
__device__ __forceinline__ void load_raw(const unsigned char* row, int V, int beta, int lane, RawBlock<DT, AL>& r) {
  constexpr int VW = Dt<DT>::VW;
  const int base = beta * BLK + lane * VW;
  if constexpr (AL) {
#pragma unroll
    for (int i = 0; i < 32 / VW; ++i) {
      const int e0 = base + i * 64 * VW;
      if constexpr (FULL) {
        const u32x4* ptr = reinterpret_cast<const u32x4*>(row + (size_t)e0 * Dt<DT>::SZ);
        const u32x4 t = NT ? __builtin_nontemporal_load(ptr) : *ptr;
        r.w[4 * i] = t.x; r.w[4 * i + 1] = t.y; r.w[4 * i + 2] = t.z; r.w[4 * i + 3] = t.w;
      } else {
        const bool in = e0 < V;
        const uint4 t = *reinterpret_cast<const uint4*>(row + (size_t)(in ? e0 : 0) * Dt<DT>::SZ);
        r.w[4 * i] = in ? t.x : NegInf<DT>::W;
        r.w[4 * i + 1] = in ? t.y : NegInf<DT>::W;
        r.w[4 * i + 2] = in ? t.z : NegInf<DT>::W;
        r.w[4 * i + 3] = in ? t.w : NegInf<DT>::W;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int e = base + (k / VW) * 64 * VW + (k % VW);
      const bool in = FULL || e < V;
      if constexpr (DT == SSD_F32) {
        const uint32_t x = reinterpret_cast<const uint32_t*>(row)[in ? e : 0];
        r.w[k] = in ? x : NegInf<DT>::W;
      } else {
        const uint32_t x = reinterpret_cast<const uint16_t*>(row)[in ? e : 0];
        r.w[k] = in ? x : NegInf<DT>::H;
      }
    }
  }
}

// Element k (static) of a packed block, decoded: the same value decode_raw
// puts in v[k].
template <int DT, bool AL>
__device__ __forceinline__ float raw_elem(const RawBlock<DT, AL>& r, int k) {
  if constexpr (DT == SSD_F32) return __uint_as_float(r.w[k]);
  if constexpr (AL) {
    const uint32_t w = r.w[k >> 1];
    if constexpr (DT == SSD_BF16) return (k & 1) ? bf16hi(w) : bf16lo(w);
    else return (k & 1) ? f16hi(w) : f16lo(w);
  } else {
    if constexpr (DT == SSD_BF16) return __uint_as_float(r.w[k] << 16);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)r.w[k]);
  }
}

template <int DT, bool AL>
__device__ __forceinline__ void decode_raw(const RawBlock<DT, AL>& r, float (&v)[32]) {
  if constexpr (AL) {
#pragma unroll
    for (int i = 0; i < 32 / Dt<DT>::VW; ++i)
      decode16<DT>(make_uint4(r.w[4 * i], r.w[4 * i + 1], r.w[4 * i + 2], r.w[4 * i + 3]), &v[i * Dt<DT>::VW]);
  } else {
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      if constexpr (DT == SSD_F32) v[k] = __uint_as_float(r.w[k]);
      else if constexpr (DT == SSD_BF16) v[k] = __uint_as_float(r.w[k] << 16);
      else v[k] = (float)__builtin_bit_cast(_Float16, (uint16_t)r.w[k]);
    }
  }
}

// Element indices fit in int32 (V <= 2^20).
template <int DT>
__device__ __forceinline__ int block_elem_index(int beta, int lane, int k) {
  constexpr int VW = Dt<DT>::VW;
  return beta * BLK + ((k / VW) * 64 + lane) * VW + (k % VW);
}

// ---------------------------------------------------------------------------
// wave64 reductions.  Inside each row of 16 lanes a butterfly of DPP moves
// (quad xor 1, quad xor 2, half-row mirror, row mirror) leaves the row's
// result in every lane; the four rows are then combined from lanes 0, 16,
// 32, 48 in a fixed order.  The whole wave must be active.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const uint64_t u = __double_as_longlong(x);
  const int lo = dpp_i<CTRL>((int)(uint32_t)u), hi = dpp_i<CTRL>((int)(uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t u) {
  const int lo = dpp_i<CTRL>((int)(uint32_t)u), hi = dpp_i<CTRL>((int)(uint32_t)(u >> 32));
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

constexpr int DPP_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_HMIR = 0x141;  // row_half_mirror
constexpr int DPP_MIR = 0x140;   // row_mirror

__device__ __forceinline__ float rl_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ double rl_d(double x, int l) {
  const uint64_t u = __double_as_longlong(x);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ uint64_t rl_u64(uint64_t u, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<DPP_XOR1>(x));
  x = fmaxf(x, dpp_f<DPP_XOR2>(x));
  x = fmaxf(x, dpp_f<DPP_HMIR>(x));
  x = fmaxf(x, dpp_f<DPP_MIR>(x));
  return fmaxf(fmaxf(rl_f(x, 0), rl_f(x, 16)), fmaxf(rl_f(x, 32), rl_f(x, 48)));
}
// Three-input maximum in one instruction (fmaxf would first quiet each
// operand that does not come from an arithmetic instruction; NaN logits are
// outside the supported domain).
__device__ __forceinline__ float fmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float wave_max3(float x) {
  x = fmax3(x, dpp_f<DPP_XOR1>(x), x);
  x = fmax3(x, dpp_f<DPP_XOR2>(x), x);
  x = fmax3(x, dpp_f<DPP_HMIR>(x), x);
  x = fmax3(x, dpp_f<DPP_MIR>(x), x);
  return fmax3(fmax3(rl_f(x, 0), rl_f(x, 16), rl_f(x, 32)), rl_f(x, 48), rl_f(x, 48));
}
__device__ __forceinline__ float wave_sum(float x) {
  x = x + dpp_f<DPP_XOR1>(x);
  x = x + dpp_f<DPP_XOR2>(x);
  x = x + dpp_f<DPP_HMIR>(x);
  x = x + dpp_f<DPP_MIR>(x);
  return (rl_f(x, 0) + rl_f(x, 16)) + (rl_f(x, 32) + rl_f(x, 48));
}
__device__ __forceinline__ double wave_sum_d(double x) {
  x = x + dpp_d<DPP_XOR1>(x);
  x = x + dpp_d<DPP_XOR2>(x);
  x = x + dpp_d<DPP_HMIR>(x);
  x = x + dpp_d<DPP_MIR>(x);
  return (rl_d(x, 0) + rl_d(x, 16)) + (rl_d(x, 32) + rl_d(x, 48));
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  x = umax64(x, dpp_u64<DPP_XOR1>(x));
  x = umax64(x, dpp_u64<DPP_XOR2>(x));
  x = umax64(x, dpp_u64<DPP_HMIR>(x));
  x = umax64(x, dpp_u64<DPP_MIR>(x));
  return umax64(umax64(rl_u64(x, 0), rl_u64(x, 16)), umax64(rl_u64(x, 32), rl_u64(x, 48)));
}
__device__ __forceinline__ int wave_min_i(int x) {
  x = min(x, dpp_i<DPP_XOR1>(x));
  x = min(x, dpp_i<DPP_XOR2>(x));
  x = min(x, dpp_i<DPP_HMIR>(x));
  x = min(x, dpp_i<DPP_MIR>(x));
  return min(min(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             min(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, (uint32_t)dpp_i<DPP_XOR1>((int)x));
  x = min(x, (uint32_t)dpp_i<DPP_XOR2>((int)x));
  x = min(x, (uint32_t)dpp_i<DPP_HMIR>((int)x));
  x = min(x, (uint32_t)dpp_i<DPP_MIR>((int)x));
  const uint32_t a = __builtin_amdgcn_readlane((int)x, 0), b = __builtin_amdgcn_readlane((int)x, 16);
  const uint32_t c = __builtin_amdgcn_readlane((int)x, 32), d = __builtin_amdgcn_readlane((int)x, 48);
  return min(min(a, b), min(c, d));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)dpp_i<DPP_XOR1>((int)x));
  x = max(x, (uint32_t)dpp_i<DPP_XOR2>((int)x));
  x = max(x, (uint32_t)dpp_i<DPP_HMIR>((int)x));
  x = max(x, (uint32_t)dpp_i<DPP_MIR>((int)x));
  const uint32_t a = __builtin_amdgcn_readlane((int)x, 0), b = __builtin_amdgcn_readlane((int)x, 16);
  const uint32_t c = __builtin_amdgcn_readlane((int)x, 32), d = __builtin_amdgcn_readlane((int)x, 48);
  return max(max(a, b), max(c, d));
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t x) {
  x = umin64(x, dpp_u64<DPP_XOR1>(x));
  x = umin64(x, dpp_u64<DPP_XOR2>(x));
  x = umin64(x, dpp_u64<DPP_HMIR>(x));
  x = umin64(x, dpp_u64<DPP_MIR>(x));
  return umin64(umin64(rl_u64(x, 0), rl_u64(x, 16)), umin64(rl_u64(x, 32), rl_u64(x, 48)));
}

// Workgroup barrier for exchanges through LDS: the fences order LDS accesses
// only, so the barrier does not wait for outstanding global loads and stores
// as __syncthreads does (a store still in flight costs a round trip to
// memory there).  Every exchange between the threads of a workgroup in these
// kernels goes through LDS.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// workgroup reductions for the epilogue kernels (EWG threads; every thread
// calls and gets the result, combined in a fixed order).  Each call site
// passes its own LDS slot of ENW entries, so one barrier per reduction
// suffices (a slot is never rewritten within a kernel, or only after a later
// barrier).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wg_max(float x, float* slot) {
  x = wave_max(x);
  if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = x;
  lds_sync();
  float m = slot[0];
#pragma unroll
  for (int k = 1; k < ENW; ++k) m = fmaxf(m, slot[k]);
  return m;
}
__device__ __forceinline__ double wg_sum_d(double x, double* slot) {
  x = wave_sum_d(x);
  if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = x;
  lds_sync();
  double t = slot[0];
#pragma unroll
  for (int k = 1; k < ENW; ++k) t += slot[k];
  return t;
}
__device__ __forceinline__ uint64_t wg_min_u64(uint64_t x, uint64_t* slot) {
  x = wave_min_u64(x);
  if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = x;
  lds_sync();
  uint64_t m = slot[0];
#pragma unroll
  for (int k = 1; k < ENW; ++k) m = umin64(m, slot[k]);
  return m;
}
__device__ __forceinline__ uint64_t wg_max_u64(uint64_t x, uint64_t* slot) {
  x = wave_max_u64(x);
  if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = x;
  lds_sync();
  uint64_t m = slot[0];
#pragma unroll
  for (int k = 1; k < ENW; ++k) m = umax64(m, slot[k]);
  return m;
}
__device__ __forceinline__ int wg_min_i(int x, int* slot) {
  x = wave_min_i(x);
  if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = x;
  lds_sync();
  int m = slot[0];
#pragma unroll
  for (int k = 1; k < ENW; ++k) m = min(m, slot[k]);
  return m;
}

// Race key of a candidate: a non-negative float key (smaller wins) in the
// high word, its index in the low word, so the unsigned minimum picks the
// smallest key and, among equal keys, the lowest index.
__device__ __forceinline__ uint64_t race_key(float key, int idx) {
  return ((uint64_t)__float_as_uint(key) << 32) | (uint32_t)idx;
}
constexpr uint64_t NO_KEY = ~0ull;

// Order-preserving key of (value desc, index asc): larger key = better.
__device__ __forceinline__ uint64_t vi_key(float v, int64_t idx) {
  uint32_t b = __float_as_uint(v + 0.0f);  // -0 -> +0
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
}
// Order-preserving 32-bit key of a float (larger float, larger key; -0 = +0).
__device__ __forceinline__ uint32_t ord_key(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float ord_val(uint32_t b) {
  return __uint_as_float((b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b);
}
__device__ __forceinline__ float key_val(uint64_t k) {
  uint32_t b = (uint32_t)(k >> 32);
  b = (b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b;
  return __uint_as_float(b);
}
__device__ __forceinline__ int64_t key_idx(uint64_t k) {
  return (int64_t)(0xFFFFFFFFu - (uint32_t)k);
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11): ten rounds of two 32x32->64-bit
// multiplies with a Weyl key schedule.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c.w ^ k1,
                   (uint32_t)p0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

enum Stream : uint32_t {
  ST_DRAFT_TOKEN = 0,
  ST_DRAFT_BLOCK = 1,
  ST_ACCEPT = 2,
  ST_BONUS_TOKEN = 3,
  ST_BONUS_BLOCK = 4,
  ST_FALLBACK = 5
};

// Four draws idx = 4c .. 4c+3 of stream `st` at (b, j).
__device__ __forceinline__ uint4 draws4(uint64_t seed, uint32_t c, uint32_t b, uint32_t j, uint32_t st) {
  return philox(make_uint4(c, b, j, st), (uint32_t)seed, (uint32_t)(seed >> 32));
}
__device__ __forceinline__ uint32_t draw1(uint64_t seed, uint32_t idx, uint32_t b, uint32_t j, uint32_t st) {
  const uint4 w = draws4(seed, idx >> 2, b, j, st);
  const uint32_t s = idx & 3u;
  return s == 0 ? w.x : s == 1 ? w.y : s == 2 ? w.z : w.w;
}
// A token in [0, V) from a word: the high half of w * V.
__device__ __forceinline__ int token_of_word(uint32_t w, int64_t V) {
  return (int)(((uint64_t)w * (uint64_t)V) >> 32);
}
// Token i of the random stand-in for sequence b's missed cache entry.
__device__ __forceinline__ int fallback_token(uint64_t seed, int b, int i, int64_t V) {
  return token_of_word(draw1(seed, (uint32_t)i, (uint32_t)b, 0u, ST_FALLBACK), V);
}
// u = ((w >> 9) + 0.5) * 2^-23: an odd multiple of 2^-24, exact in binary32.
__device__ __forceinline__ float uniform_of(uint32_t w) {
  return (float)(((w >> 9) << 1) | 1u) * 5.9604644775390625e-8f;  // 2^-24
}
// ln x (x >= 0) in double from the binary exponent and a hardware log2 of
// the mantissa rounded to binary32: absolute error about 1e-7, a few dozen
// times cheaper on the latency path than the fp64 library logarithm.
__device__ __forceinline__ double ln_fast(double x) {
  int e;
  const double f = frexp(x, &e);  // x = f 2^e, f in [0.5, 1)
  return ((double)e + (double)__builtin_amdgcn_logf((float)f)) * LN2;
}
// e^y in double from a hardware exp2 of the fractional part of y log2(e):
// relative error about 1e-7.
__device__ __forceinline__ double exp_fast(double y) {
  if (!(y > -1.0e4)) return 0.0;
  const double t = fmin(y * LOG2E, 1.0e4), k = floor(t);
  return ldexp((double)__builtin_amdgcn_exp2f((float)(t - k)), (int)k);
}

// -log2(u) = (-ln u) / ln 2 with the hardware log2 (measured within 1 ulp on
// gfx950 over every uniform this generator produces, including u near 1).
__device__ __forceinline__ float neg_log2_u(uint32_t w) { return -__builtin_amdgcn_logf(uniform_of(w)); }

}  // namespace ssd
