// gfx950 kernels of the verify-and-resample path.
//
// Every row of V logits is streamed from HBM once, in 2048-token blocks: a
// wave64 owns one block (32 elements per lane, 16-byte loads, consecutive
// lanes on consecutive 16-byte chunks) and reduces it with DPP to a block
// partial (block max M and the sum of exp((z - M)/T), or the block argmax for
// greedy rows).  A second kernel then runs one workgroup per row (or per
// sequence, for verification) over those partials: merge, exact top-F, and
// the two-level Gumbel-max draw (block by ln W + g over the partials, then
// token inside the chosen block, which is re-read), so Philox runs for about
// NB + 2048 draws per row instead of V.  The kernel boundary between the two
// makes the partials visible without any cross-workgroup synchronisation.
// Sources are cited in ssd.h.
#pragma once

#include "device.hpp"

namespace ssd {

enum Mode { M_SOFTMAX = 0, M_TOPF = 1, M_SAMPLE = 2, M_VERIFY = 3 };

constexpr int CH = 8;    // blocks per workgroup in the streaming pass (2 per wave)
constexpr int CH_R = 4;  // blocks per workgroup in the residual pass (1 per wave)
constexpr int CF = CH;   // largest top-F the streaming workgroups select locally

// What verification hands to the residual pass for one sequence.
struct SeqState {
  int need;   // 1: bonus from the residual at row kstar (T > 0, kstar < K)
  int kstar;
  float s;    // log2(e) / T
  float o_t;  // fl(-m_t * s): offset of target row kstar
  float m_t;  // max of target row kstar
  float pad;
  double L_t; // ln sum exp((z - m_t)/T) of target row kstar
};

struct Params {
  const unsigned char* x;   // logits (target rows for verification)
  const unsigned char* xd;  // draft logits (verification, residual)
  int64_t V, ld;            // ld in elements
  int64_t rows;             // rows streamed by the kernel
  int NB, nchunk;           // blocks per row, workgroups per row
  int K, B;
  const float* temp;
  int F, F_out, F_sel;
  float C;
  uint64_t seed;
  float2* part;             // block partials [rows, NB]
  uint64_t* cand;           // per-chunk top-F candidates [rows, nchunk, CF] (value bits | index << 32)
  int* cst;                 // per-chunk candidate status [rows, nchunk]: 1 ok, 0 not available
  int local_topf;           // streaming workgroups publish chunk-local top-F
  ssd_row_stats* stats;     // per-row statistics out
  float* probs;             // softmax probabilities out
  int32_t* out_idx;         // top-F indices out
  float* out_val;           // top-F values out
  int32_t* tokens;          // drafted tokens out
  float* q;                 // sigma_j(x_j) out
  const int32_t* dtok;      // drafted tokens in (verification)
  const float* dq;          // sigma_j(x_j) of the drafted tokens (verification)
  float* zcap;              // target logit at each drafted token [B, K] (workspace)
  const ssd_row_stats* dstats;
  const int32_t* dtopf;
  int ld_dtopf;
  int32_t* acc_len;
  int32_t* bonus;
  float* p_out;
  SeqState* state;
  float* rpart;             // residual block sums [B, NB]
};

struct Smem {
  Red red;
  int ncb, cnt;
  float tau;
  int nsb;
  union {
    struct {
      float M[MAX_NB];     // block maxima
      float S[MAX_NB];     // block sums
      int cblk[MAX_NB];    // candidate blocks for top-F
    } r;
    float2 stage[STAGE];   // verification: staged partials of several rows
  } u;
  float lv[CAND_CAP];      // top-F candidates (value, index)
  int li[CAND_CAP];
  float tval[MAX_F];       // top-F result, sorted
  int tidx[MAX_F];
  double es[MAX_F];        // exp2((z_s - m) * s) of the top-F set
  int sblk[MAX_F];         // top-F set members inside the sampled block
  int wcnt[ENW];
  float zwin;              // value of the token-stage winner
  float cm[CH];            // block maxima of this chunk
  float tauc;
  // verification, per row j <= K
  float vm[MAX_K1];
  double vL[MAX_K1];
  int vfmb[MAX_K1];
  int vam[MAX_K1];
  int vx[MAX_K1];
  float vq[MAX_K1];
  float vz[MAX_K1];
  int vacc[MAX_K1];
};

// ---------------------------------------------------------------------------
// streaming block partial of one block (one wave): (M, S) with M the block
// maximum and S = sum_x 2^(z_x*s + fl(-M*s)) for T > 0; for greedy rows
// (s = 0) S carries the bit pattern of the lowest index of M in the block.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float2 block_partial(const float (&v)[32], float s, int beta, int lane, int V) {
  float m0 = fmaxf(v[0], v[1]), m1 = fmaxf(v[2], v[3]);
#pragma unroll
  for (int k = 4; k < 32; k += 4) {
    m0 = fmaxf(m0, fmaxf(v[k], v[k + 1]));
    m1 = fmaxf(m1, fmaxf(v[k + 2], v[k + 3]));
  }
  const float M = wave_max(fmaxf(m0, m1));
  if (s > 0.f) {
    const float o = (M == -INFINITY) ? 0.f : -M * s;
    float a0 = __builtin_amdgcn_exp2f(fmaf(v[0], s, o)), a1 = __builtin_amdgcn_exp2f(fmaf(v[1], s, o));
    float a2 = __builtin_amdgcn_exp2f(fmaf(v[2], s, o)), a3 = __builtin_amdgcn_exp2f(fmaf(v[3], s, o));
#pragma unroll
    for (int k = 4; k < 32; k += 4) {
      a0 += __builtin_amdgcn_exp2f(fmaf(v[k], s, o));
      a1 += __builtin_amdgcn_exp2f(fmaf(v[k + 1], s, o));
      a2 += __builtin_amdgcn_exp2f(fmaf(v[k + 2], s, o));
      a3 += __builtin_amdgcn_exp2f(fmaf(v[k + 3], s, o));
    }
    return make_float2(M, wave_sum((a0 + a1) + (a2 + a3)));
  }
  int best = 0x7fffffff;
#pragma unroll
  for (int k = 31; k >= 0; --k) {
    const int idx = block_elem_index<DT>(beta, lane, k);
    if (v[k] == M && idx < V) best = idx;  // k descending: ends on the lowest index
  }
  return make_float2(M, __int_as_float(wave_min_i(best)));
}

// Exponent x (base 2) of block weight W = S * 2^x relative to row max m:
// undoes the rounding of the block offset fl(-M*s) used while streaming.
__device__ __forceinline__ double block_x(float M, float m, float s) {
  const float o = -M * s;
  const double e = (double)o + (double)M * (double)s;
  return ((double)M - (double)m) * (double)s - e;
}
__device__ __forceinline__ double block_w(float M, float S, float m, float s) {
  if (M == -INFINITY || !(S > 0.f)) return 0.0;
  return (double)S * (double)exp2f((float)block_x(M, m, s));
}
__device__ __forceinline__ double block_lnw(float M, float S, float m, float s) {
  if (M == -INFINITY || !(S > 0.f)) return -INFINITY;
  return (double)logf(S) + block_x(M, m, s) * LN2;
}

// ---------------------------------------------------------------------------
// workgroup helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wg_min_i(int x, Smem& sm) {
  x = wave_min_i(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.wcnt[threadIdx.x >> 6] = x;
  __syncthreads();
  int m = sm.wcnt[0];
  for (int k = 1; k < ENW; ++k) m = min(m, sm.wcnt[k]);
  return m;
}

// Ascending compaction of {i < n : pred(i)} into out; returns the count.
template <class Pred>
__device__ int wg_compact(int n, int* out, Smem& sm, Pred pred) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int running = 0;
  for (int base = 0; base < n; base += EWG) {
    const int i = base + threadIdx.x;
    const bool f = i < n && pred(i);
    const uint64_t m = __ballot(f);
    const int pre = __popcll(m & ((1ull << lane) - 1ull));
    __syncthreads();
    if (lane == 0) sm.wcnt[wave] = __popcll(m);
    __syncthreads();
    int off = running;
    for (int w = 0; w < wave; ++w) off += sm.wcnt[w];
    if (f) out[off + pre] = i;
    for (int w = 0; w < ENW; ++w) running += sm.wcnt[w];
  }
  __syncthreads();
  return running;
}

// Chunk-local top-F (F <= number of blocks of the chunk): the F-th largest
// block maximum tau_c bounds the chunk's F-th largest element from below, so
// the chunk's top-F are among its elements >= tau_c, which are few and are
// read from registers.  Publishes the chunk's top-F (value desc, index asc);
// status 0 (ties overflowing the list, or a chunk with fewer than F blocks)
// sends the row's epilogue to a re-read of its candidate blocks.
template <int DT>
__device__ void chunk_topf(const Params& p, int64_t row, int chunk, int b0, int b1, float M0, float M1,
                           const float (&v0)[32], const float (&v1)[32], Smem& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, V = (int)p.V, NB = p.NB, Fs = p.F_sel;
  const int nbc = min(CH, NB - chunk * CH);
  uint64_t* out = p.cand + (row * p.nchunk + chunk) * CF;
  if (Fs > nbc) {
    if (threadIdx.x == 0) p.cst[row * p.nchunk + chunk] = 0;
    return;
  }
  if (lane == 0) {
    sm.cm[wave] = b0 < NB ? M0 : -INFINITY;
    sm.cm[wave + NWAVE] = b1 < NB ? M1 : -INFINITY;
  }
  if (threadIdx.x == 0) sm.cnt = 0;
  __syncthreads();
  if (threadIdx.x < CH) {
    const float mb = sm.cm[threadIdx.x];
    int r = 0;
    for (int k = 0; k < CH; ++k) r += (sm.cm[k] > mb) || (sm.cm[k] == mb && k < (int)threadIdx.x);
    if (r == Fs - 1) sm.tauc = mb;
  }
  __syncthreads();
  const float tau = sm.tauc;
  if (b0 < NB && M0 >= tau) {
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int idx = block_elem_index<DT>(b0, lane, k);
      if (v0[k] >= tau && idx < V) {
        const int pos = atomicAdd(&sm.cnt, 1);
        if (pos < CAND_CAP) { sm.lv[pos] = v0[k]; sm.li[pos] = idx; }
      }
    }
  }
  if (b1 < NB && M1 >= tau) {
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int idx = block_elem_index<DT>(b1, lane, k);
      if (v1[k] >= tau && idx < V) {
        const int pos = atomicAdd(&sm.cnt, 1);
        if (pos < CAND_CAP) { sm.lv[pos] = v1[k]; sm.li[pos] = idx; }
      }
    }
  }
  __syncthreads();
  const int n = sm.cnt;
  if (n > CAND_CAP) {
    if (threadIdx.x == 0) p.cst[row * p.nchunk + chunk] = 0;
    return;
  }
  for (int i = threadIdx.x; i < n; i += WG) {
    const float vi = sm.lv[i];
    const int ii = sm.li[i];
    int r = 0;
    for (int k = 0; k < n; ++k) r += (sm.lv[k] > vi) || (sm.lv[k] == vi && sm.li[k] < ii);
    if (r < Fs)
      out[r] = ((uint64_t)(uint32_t)ii << 32) | __float_as_uint(vi);
  }
  if (threadIdx.x == 0) p.cst[row * p.nchunk + chunk] = 1;
}

// Row top-F from the chunks' published lists (all status 1): the union of
// the chunks' top-F holds the row's top-F.  Returns false if a chunk could
// not publish (the caller then re-reads candidate blocks).
__device__ bool merge_chunk_topf(const Params& p, int64_t row, Smem& sm) {
  const int Fs = p.F_sel, nc = p.nchunk;
  if (!p.local_topf) return false;
  const int n = nc * Fs;
  // status and candidates are loaded together (one round trip)
  int ok = 1;
  uint64_t e[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = threadIdx.x + k * EWG;
    e[k] = i < n ? p.cand[(row * nc + i / Fs) * CF + i % Fs] : 0;
  }
  for (int c = threadIdx.x; c < nc; c += EWG) ok &= p.cst[row * nc + c];
  if (n > 2 * EWG || wg_min_i(ok, sm) == 0) return false;
  // keep entries >= the Fs-th largest block maximum (always includes the top-Fs)
  const float tau = sm.tau;
  if (threadIdx.x == 0) sm.cnt = 0;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = threadIdx.x + k * EWG;
    const float v = __uint_as_float((uint32_t)e[k]);
    if (i < n && v >= tau) {
      const int pos = atomicAdd(&sm.cnt, 1);
      if (pos < CAND_CAP) { sm.lv[pos] = v; sm.li[pos] = (int)(e[k] >> 32); }
    }
  }
  __syncthreads();
  const int m = sm.cnt;
  if (m > CAND_CAP) return false;
  for (int i = threadIdx.x; i < m; i += EWG) {
    const float vi = sm.lv[i];
    const int ii = sm.li[i];
    int r = 0;
    for (int k = 0; k < m; ++k) r += (sm.lv[k] > vi) || (sm.lv[k] == vi && sm.li[k] < ii);
    if (r < Fs) { sm.tval[r] = vi; sm.tidx[r] = ii; }
  }
  __syncthreads();
  return true;
}

// Row partials -> sm.u.r.M / sm.u.r.S (all threads).
__device__ __forceinline__ void load_partials(const float2* pr, int NB, Smem& sm) {
  for (int be = threadIdx.x; be < NB; be += EWG) {
    const float2 v = pr[be];
    sm.u.r.M[be] = v.x;
    sm.u.r.S[be] = v.y;
  }
  __syncthreads();
}

// Lowest index of value m inside block beta (one wave).
template <int DT, bool AL>
__device__ int wave_first_eq(const unsigned char* rp, int64_t V, int beta, float m) {
  const int lane = threadIdx.x & 63;
  float v[32];
  load_block<DT, AL>(rp, V, beta, lane, v);
  int best = 0x7fffffff;
#pragma unroll
  for (int k = 31; k >= 0; --k) {
    const int idx = (int)block_elem_index<DT>(beta, lane, k);
    if (v[k] == m && idx < V) best = min(best, idx);
  }
  return wave_min_i(best);
}

// Exact top-Fsel of a row into sm.tval / sm.tidx (value desc, index asc).
// The Fsel-th largest block maximum tau bounds the Fsel-th largest element
// from below, so every top element lies in a block with maximum >= tau; only
// those blocks are re-read, and only their elements >= tau are ranked.
// sm.tau = the Fsel-th largest block maximum, counted with multiplicity
// (-inf if NB <= Fsel): wave 0 removes the maximum Fsel times.
__device__ void block_max_threshold(int NB, int Fsel, Smem& sm) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    constexpr int PL = MAX_NB / 64;
    float v[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) v[i] = (lane + 64 * i < NB) ? sm.u.r.M[lane + 64 * i] : -INFINITY;
    float tau = -INFINITY;
    if (NB > Fsel) {
      for (int r = 0; r < Fsel; ++r) {
        float lm = v[0];
#pragma unroll
        for (int i = 1; i < PL; ++i) lm = fmaxf(lm, v[i]);
        const float m = wave_max(lm);
        const uint64_t bal = __ballot(lm == m);
        if (lane == (int)__builtin_ctzll(bal)) {
          bool done = false;
#pragma unroll
          for (int i = 0; i < PL; ++i)
            if (!done && v[i] == m) {
              v[i] = -INFINITY;
              done = true;
            }
        }
        tau = m;
      }
    }
    if (lane == 0) sm.tau = tau;
  }
  __syncthreads();
}

template <int DT, bool AL>
__device__ void wg_topf(const unsigned char* rp, int64_t V, int NB, int Fsel, Smem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  block_max_threshold(NB, Fsel, sm);
  const float tau = sm.tau;
  const int ncb = wg_compact(NB, sm.u.r.cblk, sm, [&](int be) { return sm.u.r.M[be] >= tau; });
  if (tid == 0) sm.cnt = 0;
  __syncthreads();
  for (int c = wave; c < ncb; c += ENW) {
    const int be = sm.u.r.cblk[c];
    float v[32];
    load_block<DT, AL>(rp, V, be, lane, v);
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int idx = block_elem_index<DT>(be, lane, k);
      if (v[k] >= tau && idx < V) {
        const int pos = atomicAdd(&sm.cnt, 1);
        if (pos < CAND_CAP) {
          sm.lv[pos] = v[k];
          sm.li[pos] = idx;
        }
      }
    }
  }
  __syncthreads();
  const int n = sm.cnt;
  if (n <= CAND_CAP) {
    for (int i = tid; i < n; i += EWG) {
      const float vi = sm.lv[i];
      const int ii = sm.li[i];
      int r = 0;
      for (int k = 0; k < n; ++k) {
        const float vk = sm.lv[k];
        r += (vk > vi) || (vk == vi && sm.li[k] < ii);
      }
      if (r < Fsel) {
        sm.tval[r] = vi;
        sm.tidx[r] = ii;
      }
    }
  } else {
    // Many ties at the threshold: pick the best key below the previous one,
    // Fsel times, over the candidate blocks.
    uint64_t prev = ~0ull;
    constexpr int VW = Dt<DT>::VW;
    for (int r = 0; r < Fsel; ++r) {
      uint64_t best = 0;
      for (int c = wave; c < ncb; c += ENW) {
        const int be = sm.u.r.cblk[c];
#pragma unroll 1
        for (int i = 0; i < 32 / VW; ++i) {
          const int e0 = be * BLK + (i * 64 + lane) * VW;
          float v[VW];
          load_chunk<DT, AL>(rp, (int)V, e0, v);
#pragma unroll
          for (int e = 0; e < VW; ++e) {
            if (v[e] >= tau && e0 + e < V) {
              const uint64_t key = vi_key(v[e], e0 + e);
              if (key < prev) best = umax64(best, key);
            }
          }
        }
      }
      best = wg_max_u64(best, sm.red);
      if (tid == 0) {
        sm.tval[r] = key_val(best);
        sm.tidx[r] = (int)key_idx(best);
      }
      prev = best;
    }
  }
  __syncthreads();
}

// Block stage of the two-level sampler: argmax over blocks of lnw(be) + g.
template <class LnW>
__device__ Arg block_stage(int NB, uint64_t seed, int b, int j, uint32_t st, Smem& sm, LnW lnw) {
  Arg best{-INFINITY, (int64_t)0x7fffffff};
  for (int be = threadIdx.x; be < NB; be += EWG) {
    const double l = lnw(be);
    if (l > -INFINITY) {
      const double sc = l + (double)gumbel_of(draw1(seed, (uint32_t)be, (uint32_t)b, (uint32_t)j, st));
      best = better(best, Arg{sc, be});
    }
  }
  return wg_argmax(best, sm.red);
}

// Four consecutive elements x0..x0+3 of a row (x0 a multiple of 4); past V
// reads as -inf.
template <int DT>
__device__ __forceinline__ void load4(const unsigned char* rp, int V, int x0, float (&o)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool in = x0 + e < V;
    const float x = load_elem<DT>(rp, in ? x0 + e : 0);
    o[e] = in ? x : -INFINITY;
  }
}

static_assert(BLK == 4 * EWG, "the token stages give each epilogue thread four tokens");

// Token stage: argmax over x in block beta of score(z1[x], z2[x], x) + g(x);
// score returns -inf to exclude a token.  rp2 may alias rp1.  The winner's
// z1 value is left in sm.zwin.
template <int DT, bool AL, class Score>
__device__ Arg token_stage(const unsigned char* rp1, const unsigned char* rp2, int64_t V, int beta,
                           uint64_t seed, int b, int j, uint32_t st, Smem& sm, Score score) {
  const int x0 = beta * BLK + 4 * (int)threadIdx.x;
  float z1[4], z2[4];
  load4<DT>(rp1, (int)V, x0, z1);
  load4<DT>(rp2, (int)V, x0, z2);
  Arg best{-INFINITY, (int64_t)0x7fffffff};
  float zb = 0.f;
  if (x0 < V) {
    const uint4 wa = draws4(seed, (uint32_t)(x0 >> 2), (uint32_t)b, (uint32_t)j, st);
    const uint32_t w[4] = {wa.x, wa.y, wa.z, wa.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int x = x0 + e;
      if (x < V) {
        const double sc = score(z1[e], z2[e], x);
        if (sc > -INFINITY) {
          const Arg a{sc + (double)gumbel_of(w[e]), x};
          if (better(best, a).i == a.i) zb = z1[e];
          best = better(best, a);
        }
      }
    }
  }
  const Arg r = wg_argmax(best, sm.red);
  if (best.i == r.i) sm.zwin = zb;
  __syncthreads();
  return r;
}

// Members of the first F top entries that fall in block beta -> sm.sblk.
__device__ __forceinline__ void s_in_block(int F, int beta, Smem& sm) {
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    for (int f = 0; f < F; ++f)
      if (sm.tidx[f] / BLK == beta) sm.sblk[n++] = sm.tidx[f];
    sm.nsb = n;
  }
  __syncthreads();
}
__device__ __forceinline__ bool in_sblk(int x, const Smem& sm) {
  for (int k = 0; k < sm.nsb; ++k)
    if (sm.sblk[k] == x) return true;
  return false;
}

// -ln(u) of the 24-bit uniform of word w, accurate near u = 1 (log1p of the
// exact u - 1).
__device__ __forceinline__ float neglog_u(uint32_t w) {
  const float u = uniform_of(w);
  return u > 0.5f ? -log1pf(u - 1.0f) : -logf(u);
}

// Token stage for weights w_x = 2^(a_x), a_x = (z_x - m) * s + c2 * [x in S]
// (s = log2(e)/T, c2 = log2 C): argmax of ln w_x + g(x) taken as the argmin
// of -ln(u_x) * 2^(-a_x), the same decision with one log and one exp per
// token.  Ties go to the lower index; the winner's logit is left in sm.zwin.
template <int DT, bool AL>
__device__ Arg token_stage_w(const unsigned char* rp, int V, int beta, uint64_t seed, int b, int j, uint32_t st,
                             float m, float s, float c2, Smem& sm) {
  const int x0 = beta * BLK + 4 * (int)threadIdx.x;
  float z[4];
  load4<DT>(rp, V, x0, z);
  Arg best{-INFINITY, (int64_t)0x7fffffff};
  float zb = 0.f;
  if (x0 < V) {
    const uint4 wa = draws4(seed, (uint32_t)(x0 >> 2), (uint32_t)b, (uint32_t)j, st);
    const uint32_t w[4] = {wa.x, wa.y, wa.z, wa.w};
    const float om = -m * s;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int x = x0 + e;
      if (x < V && z[e] > -INFINITY) {
        const float a = fmaf(z[e], s, om) + (in_sblk(x, sm) ? c2 : 0.f);
        const float key = neglog_u(w[e]) * __builtin_amdgcn_exp2f(-a);
        const Arg c{-(double)key, x};
        if (better(best, c).i == c.i) {
          best = c;
          zb = z[e];
        }
      }
    }
  }
  const Arg r = wg_argmax(best, sm.red);
  if (best.i == r.i) sm.zwin = zb;
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// epilogues
// ---------------------------------------------------------------------------
template <int DT, bool AL>
__device__ void epi_softmax(const Params& p, int64_t row, Smem& sm) {
  const float T = p.temp[row];
  const bool greedy = !(T > 0.f);
  const float s = greedy ? 0.f : (float)(LOG2E / (double)T);
  const unsigned char* rp = p.x + row * p.ld * Dt<DT>::SZ;
  load_partials(p.part + row * p.NB, p.NB, sm);
  float lm = -INFINITY;
  for (int be = threadIdx.x; be < p.NB; be += EWG) lm = fmaxf(lm, sm.u.r.M[be]);
  const float m = wg_max(lm, sm.red);
  int fb = 0x7fffffff;
  double w = 0.0;
  for (int be = threadIdx.x; be < p.NB; be += EWG) {
    if (sm.u.r.M[be] == m) fb = min(fb, be);
    if (!greedy) w += block_w(sm.u.r.M[be], sm.u.r.S[be], m, s);
  }
  fb = min(wg_min_i(fb, sm), p.NB - 1);  // (a NaN row matches no block)
  const double tot = wg_sum_d(w, sm.red);
  if (threadIdx.x < 64) {
    // greedy rows carry the block argmax in their partial; others re-read the block
    const int am = greedy ? __float_as_int(sm.u.r.S[fb]) : wave_first_eq<DT, AL>(rp, p.V, fb, m);
    if (threadIdx.x == 0) {
      ssd_row_stats st;
      st.lse = greedy ? 0.0 : log(tot);
      st.max = m;
      st.argmax = am;
      p.stats[row] = st;
    }
  }
}

template <int DT, bool AL>
__device__ void epi_topf(const Params& p, int64_t row, Smem& sm) {
  const unsigned char* rp = p.x + row * p.ld * Dt<DT>::SZ;
  load_partials(p.part + row * p.NB, p.NB, sm);
  block_max_threshold(p.NB, p.F_sel, sm);
  if (!merge_chunk_topf(p, row, sm)) wg_topf<DT, AL>(rp, p.V, p.NB, p.F, sm);
  for (int r = threadIdx.x; r < p.F; r += EWG) {
    p.out_idx[row * p.F + r] = sm.tidx[r];
    if (p.out_val) p.out_val[row * p.F + r] = sm.tval[r];
  }
}

template <int DT, bool AL>
__device__ void epi_sample(const Params& p, int64_t row, Smem& sm) {
  const int K1 = p.K + 1;
  const int b = (int)(row / K1), j = (int)(row % K1);
  const float T = p.temp[b];
  const bool greedy = !(T > 0.f);
  const float s = greedy ? 0.f : (float)(LOG2E / (double)T);
  const double invT = greedy ? 0.0 : 1.0 / (double)T;
  const double lnC = log((double)p.C);
  const unsigned char* rp = p.x + row * p.ld * Dt<DT>::SZ;
  const int NB = p.NB;
  load_partials(p.part + row * NB, NB, sm);
  float lm = -INFINITY;
  for (int be = threadIdx.x; be < NB; be += EWG) lm = fmaxf(lm, sm.u.r.M[be]);
  const float m = wg_max(lm, sm.red);
  double w = 0.0;
  if (!greedy)
    for (int be = threadIdx.x; be < NB; be += EWG) w += block_w(sm.u.r.M[be], sm.u.r.S[be], m, s);
  const double tot0 = wg_sum_d(w, sm.red);
  block_max_threshold(NB, p.F_sel, sm);
  if (!merge_chunk_topf(p, row, sm)) wg_topf<DT, AL>(rp, p.V, NB, p.F_sel, sm);
  const int am = sm.tidx[0];
  // sigma_{F,C}: the first F of the top list form S; their weights
  if (!greedy && threadIdx.x < p.F)
    sm.es[threadIdx.x] = exp2(((double)sm.tval[threadIdx.x] - (double)m) * (double)s);
  __syncthreads();
  double zs = 0.0;
  for (int f = 0; f < p.F; ++f) zs += sm.es[f];
  const double totc = greedy ? 1.0 : (tot0 - zs) + (double)p.C * zs;
  const double lse = greedy ? 0.0 : log(totc);
  if (threadIdx.x == 0) {
    ssd_row_stats st;
    st.lse = lse;
    st.max = m;
    st.argmax = am;
    p.stats[row] = st;
  }
  for (int r = threadIdx.x; r < p.F_out; r += EWG) {
    if (p.out_idx) p.out_idx[row * p.F_out + r] = sm.tidx[r];
    if (p.out_val) p.out_val[row * p.F_out + r] = sm.tval[r];
  }
  if (j == p.K) return;  // row K only predicts the bonus after K acceptances
  if (greedy) {
    if (threadIdx.x == 0) {
      p.tokens[b * p.K + j] = am;
      p.q[b * p.K + j] = 1.0f;
    }
    return;
  }
  const int F = p.F;
  const float C = p.C;
  const Arg bs = block_stage(NB, p.seed, b, j, ST_DRAFT_BLOCK, sm, [&](int be) -> double {
    double corr = 0.0;
    for (int f = 0; f < F; ++f)
      if (sm.tidx[f] / BLK == be) corr += sm.es[f];
    if (corr == 0.0) return block_lnw(sm.u.r.M[be], sm.u.r.S[be], m, s);
    const double W = block_w(sm.u.r.M[be], sm.u.r.S[be], m, s);
    const double Wc = fmax(W - corr, 0.0) + (double)C * corr;
    return Wc > 0.0 ? log(Wc) : -INFINITY;
  });
  const int beta = bs.i < NB ? (int)bs.i : 0;  // no block of mass only for invalid rows
  s_in_block(F, beta, sm);
  const Arg ts = token_stage_w<DT, AL>(rp, (int)p.V, beta, p.seed, b, j, ST_DRAFT_TOKEN, m, s,
                                       (float)(lnC * LOG2E), sm);
  if (threadIdx.x == 0) {
    const int x = ts.i < p.V ? (int)ts.i : 0;
    const float z = sm.zwin;
    bool inS = false;
    for (int f = 0; f < F; ++f) inS |= (sm.tidx[f] == x);
    const double lq = ((double)z - (double)m) * invT + (inS ? lnC : 0.0) - lse;
    p.tokens[b * p.K + j] = x;
    p.q[b * p.K + j] = (float)exp(lq);
  }
}

template <int DT, bool AL>
__device__ void epi_verify(const Params& p, int b, Smem& sm) {
  const int K = p.K, K1 = K + 1, NB = p.NB, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const float T = p.temp[b];
  const bool greedy = !(T > 0.f);
  const float s = greedy ? 0.f : (float)(LOG2E / (double)T);
  const double invT = greedy ? 0.0 : 1.0 / (double)T;
  const int64_t r0 = (int64_t)b * K1;
  const int64_t rs = p.ld * Dt<DT>::SZ;
  // per-position inputs: drafted token, sigma_j(x_j), and the target logit at
  // x_j captured by the streaming pass
  if (tid < K) {
    sm.vx[tid] = p.dtok[b * K + tid];
    sm.vq[tid] = p.dq[b * K + tid];
    sm.vz[tid] = p.zcap[b * K + tid];
  }
  // merge the partials of rows 0..K, several rows per staging round
  const int rpg = max(1, STAGE / NB);
  for (int g0 = 0; g0 < K1; g0 += rpg) {
    const int n = min(rpg, K1 - g0);
    __syncthreads();
    const float2* src = p.part + (r0 + g0) * NB;
    float2 t[STAGE / EWG];
#pragma unroll
    for (int k = 0; k < STAGE / EWG; ++k) {
      const int i = tid + k * EWG;
      t[k] = i < n * NB ? src[i] : make_float2(0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < STAGE / EWG; ++k)
      if (tid + k * EWG < n * NB) sm.u.stage[tid + k * EWG] = t[k];
    __syncthreads();
    for (int jj = wave; jj < n; jj += ENW) {
      float lm = -INFINITY;
      for (int be = lane; be < NB; be += 64) lm = fmaxf(lm, sm.u.stage[jj * NB + be].x);
      const float m = wave_max(lm);
      int fb = 0x7fffffff;
      double w = 0.0;
      for (int be = lane; be < NB; be += 64) {
        const float2 v = sm.u.stage[jj * NB + be];
        if (v.x == m) fb = min(fb, be);
        if (!greedy) w += block_w(v.x, v.y, m, s);
      }
      fb = min(wave_min_i(fb), NB - 1);
      w = wave_sum_d(w);
      if (lane == 0) {
        sm.vm[g0 + jj] = m;
        sm.vL[g0 + jj] = greedy ? 0.0 : log(w);
        sm.vfmb[g0 + jj] = fb;
        // greedy rows carry the block argmax in their partial
        sm.vam[g0 + jj] = greedy ? __float_as_int(sm.u.stage[jj * NB + fb].y) : -1;
      }
    }
  }
  __syncthreads();
  // argmax of the T > 0 rows is only needed for the optional statistics
  if (!greedy && p.stats)
    for (int j = wave; j < K1; j += ENW) {
      const int am = wave_first_eq<DT, AL>(p.x + (r0 + j) * rs, p.V, sm.vfmb[j], sm.vm[j]);
      if (lane == 0) sm.vam[j] = am;
    }
  // acceptance decisions, p_j(x_j) for every position
  if (tid < K) {
    const int j = tid, x = sm.vx[j];
    const bool ok = x >= 0 && x < p.V;
    bool acc = false;
    double pj = 0.0;
    if (ok) {
      if (greedy) {
        acc = (x == sm.vam[j]);
        pj = acc ? 1.0 : 0.0;
      } else {
        const float zt = sm.vz[j];
        pj = exp(((double)zt - (double)sm.vm[j]) * invT - sm.vL[j]);
        const double q = (double)sm.vq[j];
        const double rho = q > 0.0 ? pj / q : (pj > 0.0 ? INFINITY : 0.0);
        const float u = uniform_of(draw1(p.seed, 0u, (uint32_t)b, (uint32_t)j, ST_ACCEPT));
        acc = (double)u < rho;
      }
    }
    p.p_out[b * K + j] = (float)pj;
    sm.vacc[j] = acc ? 1 : 0;
  }
  __syncthreads();
  int ks = K;
  for (int j = 0; j < K; ++j)
    if (!sm.vacc[j]) {
      ks = j;
      break;
    }
  if (p.stats && tid < K1) {
    ssd_row_stats st;
    st.lse = sm.vL[tid];
    st.max = sm.vm[tid];
    st.argmax = sm.vam[tid];
    p.stats[r0 + tid] = st;
  }
  if (tid == 0) p.acc_len[b] = ks;
  SeqState ss{};
  if (greedy) {
    if (tid == 0) {
      p.bonus[b] = sm.vam[ks];
      p.state[b] = ss;
    }
    return;
  }
  if (ks < K) {
    if (tid == 0) {
      const float mt = sm.vm[ks];
      ss.need = 1;
      ss.kstar = ks;
      ss.s = s;
      ss.o_t = -mt * s;
      ss.m_t = mt;
      ss.L_t = sm.vL[ks];
      p.state[b] = ss;
    }
    return;
  }
  // all K accepted: bonus ~ p_K
  if (tid == 0) p.state[b] = ss;
  const unsigned char* rp = p.x + (r0 + K) * rs;
  __syncthreads();
  load_partials(p.part + (r0 + K) * NB, NB, sm);
  const float m = sm.vm[K];
  const Arg bs = block_stage(NB, p.seed, b, K, ST_BONUS_BLOCK, sm,
                             [&](int be) { return block_lnw(sm.u.r.M[be], sm.u.r.S[be], m, s); });
  if (tid == 0) sm.nsb = 0;
  __syncthreads();
  const Arg ts = token_stage_w<DT, AL>(rp, (int)p.V, bs.i < NB ? (int)bs.i : 0, p.seed, b, K, ST_BONUS_TOKEN, m, s,
                                       0.f, sm);
  if (tid == 0) p.bonus[b] = ts.i < p.V ? (int)ts.i : 0;
}

template <int DT, bool AL>
__device__ void epi_residual(const Params& p, int b, const SeqState& ss, Smem& sm) {
  const int K1 = p.K + 1, NB = p.NB, ks = ss.kstar;
  const int64_t row = (int64_t)b * K1 + ks;
  const int64_t rs = p.ld * Dt<DT>::SZ;
  const unsigned char* rt = p.x + row * rs;
  const unsigned char* rd = p.xd + row * rs;
  const float T = p.temp[b];
  const double invT = 1.0 / (double)T;
  const double lnC = log((double)p.C);
  for (int be = threadIdx.x; be < NB; be += EWG) sm.u.r.S[be] = *(p.rpart + (int64_t)b * NB + be);
  if (threadIdx.x < p.F) sm.tidx[threadIdx.x] = p.dtopf[row * p.ld_dtopf + threadIdx.x];
  __syncthreads();
  double w = 0.0;
  for (int be = threadIdx.x; be < NB; be += EWG) w += (double)sm.u.r.S[be];
  const double tot = wg_sum_d(w, sm.red);
  const bool res = tot > 0.0;
  if (!res) load_partials(p.part + row * NB, NB, sm);  // no residual mass: sample p_k*
  const ssd_row_stats ds = p.dstats[row];
  const float mt = ss.m_t, md = ds.max, s = ss.s;
  const double Lt = ss.L_t, Ld = ds.lse;
  const Arg bs = block_stage(NB, p.seed, b, ks, ST_BONUS_BLOCK, sm, [&](int be) -> double {
    if (res) return sm.u.r.S[be] > 0.f ? log((double)sm.u.r.S[be]) : -INFINITY;
    return block_lnw(sm.u.r.M[be], sm.u.r.S[be], mt, s);
  });
  const int beta = bs.i < NB ? (int)bs.i : 0;
  s_in_block(p.F, beta, sm);
  // residual score: ln r = a + ln(-expm1(d)), d = ln sigma - ln p, r > 0 iff d < 0
  const Arg tr = token_stage<DT, AL>(rt, rd, p.V, beta, p.seed, b, ks, ST_BONUS_TOKEN, sm,
                                     [&](float zt, float zd, int x) -> double {
                                       if (zt == -INFINITY) return -INFINITY;
                                       const double a = ((double)zt - (double)mt) * invT - Lt;
                                       if (!res) return a;
                                       if (zd == -INFINITY) return a;
                                       const double bb =
                                           ((double)zd - (double)md) * invT + (in_sblk(x, sm) ? lnC : 0.0) - Ld;
                                       const double d = bb - a;
                                       if (!(d < 0.0)) return -INFINITY;
                                       return a + (double)logf(-expm1f((float)d));
                                     });
  int bonus = (int)tr.i;
  if (tr.s == -INFINITY) {  // chosen block had mass only through rounding: use p there
    if (threadIdx.x == 0) sm.nsb = 0;
    __syncthreads();
    const Arg tp = token_stage_w<DT, AL>(rt, (int)p.V, beta, p.seed, b, ks, ST_BONUS_TOKEN, mt, s, 0.f, sm);
    bonus = (int)tp.i;
  }
  if (threadIdx.x == 0) p.bonus[b] = (bonus >= 0 && bonus < p.V) ? bonus : 0;
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------
template <int DT, bool AL, int MODE>
__global__ __launch_bounds__(WG, (MODE == M_SAMPLE || MODE == M_TOPF) ? 5 : 6) void k_stream(Params p) {
  __shared__ Smem sm;
  const int item = blockIdx.x;
  const int64_t row = item / p.nchunk;
  const int chunk = item - (int)(row * p.nchunk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K1 = p.K + 1;
  float T = 0.f;
  if constexpr (MODE == M_SOFTMAX) T = p.temp[row];
  if constexpr (MODE == M_SAMPLE || MODE == M_VERIFY) T = p.temp[row / K1];
  const float s = (T > 0.f) ? (float)(LOG2E / (double)T) : 0.f;
  const unsigned char* rp = p.x + row * p.ld * Dt<DT>::SZ;
  const int V = (int)p.V, NB = p.NB;
  const int b0 = chunk * CH + wave, b1 = b0 + NWAVE;
  int xj = -1;  // verification: drafted token of this target row (j < K)
  if constexpr (MODE == M_VERIFY) {
    const int j = (int)(row % K1);
    if (j < p.K) xj = p.dtok[(row / K1) * p.K + j];
  }
  float v0[32], v1[32];
  if ((chunk + 1) * CH * BLK <= V) {
    // every block of this chunk is full: all loads in flight together
    load_block_full<DT, AL>(rp, b0, lane, v0);
    load_block_full<DT, AL>(rp, b1, lane, v1);
    const float2 r0 = block_partial<DT>(v0, s, b0, lane, V);
    const float2 r1 = block_partial<DT>(v1, s, b1, lane, V);
    if (lane == 0) {
      p.part[row * NB + b0] = r0;
      p.part[row * NB + b1] = r1;
    }
    if constexpr (MODE == M_SAMPLE || MODE == M_TOPF)
      if (p.local_topf) chunk_topf<DT>(p, row, chunk, b0, b1, r0.x, r1.x, v0, v1, sm);
  } else {
    // the chunk holding the ragged end of the row
    load_block<DT, AL>(rp, V, min(b0, NB - 1), lane, v0);
    load_block<DT, AL>(rp, V, min(b1, NB - 1), lane, v1);
    const float2 r0 = block_partial<DT>(v0, s, min(b0, NB - 1), lane, V);
    const float2 r1 = block_partial<DT>(v1, s, min(b1, NB - 1), lane, V);
    if (lane == 0 && b0 < NB) p.part[row * NB + b0] = r0;
    if (lane == 0 && b1 < NB) p.part[row * NB + b1] = r1;
    if constexpr (MODE == M_SAMPLE || MODE == M_TOPF)
      if (p.local_topf) chunk_topf<DT>(p, row, chunk, b0, b1, r0.x, r1.x, v0, v1, sm);
  }
  if constexpr (MODE == M_VERIFY) {
    // the workgroup whose chunk holds x_j hands its target logit to the epilogue
    if (xj >= 0 && xj < V && xj / (CH * BLK) == chunk && threadIdx.x == 0)
      p.zcap[(row / K1) * p.K + (row % K1)] = load_elem<DT>(rp, xj);
  }
}

// One workgroup per row (per sequence for verification) over the partials.
template <int DT, bool AL, int MODE>
__global__ __launch_bounds__(EWG) void k_epi(Params p) {
  __shared__ Smem sm;
  const int g = blockIdx.x;
  if constexpr (MODE == M_VERIFY) epi_verify<DT, AL>(p, g, sm);
  if constexpr (MODE == M_SOFTMAX) epi_softmax<DT, AL>(p, g, sm);
  if constexpr (MODE == M_TOPF) epi_topf<DT, AL>(p, g, sm);
  if constexpr (MODE == M_SAMPLE) epi_sample<DT, AL>(p, g, sm);
}

// Residual pass for sequences rejected at k* < K: block sums of
// max(0, p - sigma) over target row k* and draft row k*, in the target's
// units scaled by exp(L_t) 2^(e_t) (a constant per sequence).
template <int DT, bool AL>
__global__ __launch_bounds__(WG, 6) void k_residual(Params p) {
  __shared__ Smem sm;
  const int item = blockIdx.x;
  const int b = item / p.nchunk;
  const int chunk = item - b * p.nchunk;
  const SeqState ss = p.state[b];
  if (!ss.need) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K1 = p.K + 1;
  const int64_t row = (int64_t)b * K1 + ss.kstar;
  const int64_t rs = p.ld * Dt<DT>::SZ;
  const unsigned char* rt = p.x + row * rs;
  const unsigned char* rd = p.xd + row * rs;
  if (threadIdx.x < p.F) sm.tidx[threadIdx.x] = p.dtopf[row * p.ld_dtopf + threadIdx.x];
  // scale of the draft term in the target's units: 2^(e_t - e_d) exp(L_t - L_d)
  const ssd_row_stats ds = p.dstats[row];
  const float od = -ds.max * ss.s;
  const double et = (double)ss.o_t + (double)ss.m_t * (double)ss.s;
  const double ed = (double)od + (double)ds.max * (double)ss.s;
  const float kf = (float)(exp2(et - ed) * exp(ss.L_t - ds.lse));
  __syncthreads();
  const int be = chunk * CH_R + wave;
  if (be < p.NB) {
    float vt[32], vd[32];
    if ((be + 1) * BLK <= (int)p.V) {
      load_block_full<DT, AL>(rt, be, lane, vt);
      load_block_full<DT, AL>(rd, be, lane, vd);
    } else {
      load_block<DT, AL>(rt, (int)p.V, be, lane, vt);
      load_block<DT, AL>(rd, (int)p.V, be, lane, vd);
    }
    const float s = ss.s, ot = ss.o_t, nk = -kf;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int k = 0; k < 32; k += 2) {
      const float e1 = __builtin_amdgcn_exp2f(fmaf(vt[k], s, ot));
      const float e2 = __builtin_amdgcn_exp2f(fmaf(vd[k], s, od));
      const float f1 = __builtin_amdgcn_exp2f(fmaf(vt[k + 1], s, ot));
      const float f2 = __builtin_amdgcn_exp2f(fmaf(vd[k + 1], s, od));
      a0 += fmaxf(fmaf(nk, e2, e1), 0.f);
      a1 += fmaxf(fmaf(nk, f2, f1), 0.f);
    }
    float R = wave_sum(a0 + a1);
    // members of the draft's top-F set in this block carry the factor C
    for (int f = 0; f < p.F; ++f) {
      const int x = sm.tidx[f];
      if (x >= 0 && x < p.V && x / BLK == be) {
        const float zt = load_elem<DT>(rt, x), zd = load_elem<DT>(rd, x);
        const float e1 = __builtin_amdgcn_exp2f(fmaf(zt, s, ot));
        const float e2 = __builtin_amdgcn_exp2f(fmaf(zd, s, od));
        R += fmaxf(fmaf(nk * p.C, e2, e1), 0.f) - fmaxf(fmaf(nk, e2, e1), 0.f);
      }
    }
    if (lane == 0) p.rpart[(int64_t)b * p.NB + be] = fmaxf(R, 0.f);
  }
}

template <int DT, bool AL>
__global__ __launch_bounds__(EWG) void k_residual_epi(Params p) {
  __shared__ Smem sm;
  const int b = blockIdx.x;
  const SeqState ss = p.state[b];
  if (!ss.need) return;
  epi_residual<DT, AL>(p, b, ss, sm);
}

// Dense probabilities for ssd_softmax_t (after the statistics kernel).
template <int DT, bool AL>
__global__ __launch_bounds__(WG) void k_probs(Params p) {
  const int item = blockIdx.x;
  const int64_t row = item / p.nchunk;
  const int chunk = item - (int)(row * p.nchunk);
  const float T = p.temp[row];
  const ssd_row_stats st = p.stats[row];
  const unsigned char* rp = p.x + row * p.ld * Dt<DT>::SZ;
  float* out = p.probs + row * p.V;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int be = chunk * NWAVE + wave;
  if (be >= p.NB) return;
  if (!(T > 0.f)) {
    for (int k = threadIdx.x & 63; k < BLK; k += 64) {
      const int64_t x = (int64_t)be * BLK + k;
      if (x < p.V) out[x] = (x == st.argmax) ? 1.f : 0.f;
    }
    return;
  }
  const float s = (float)(LOG2E / (double)T);
  const float o = (float)(-(double)st.max * (double)s - st.lse * LOG2E);
  float v[32];
  load_block<DT, AL>(rp, p.V, be, lane, v);
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int64_t x = block_elem_index<DT>(be, lane, k);
    if (x < p.V) out[x] = __builtin_amdgcn_exp2f(fmaf(v[k], s, o));
  }
}

// One wave per sequence: find bonus among depth k*'s keys (lowest slot).
__global__ __launch_bounds__(WG) void k_lookup(const int32_t* keys, const int32_t* off, const int32_t* payload,
                                               int B, int K, int Bgt, const int32_t* acc, const int32_t* bonus,
                                               int32_t* hit, int32_t* slot, int32_t* toks) {
  const int b = blockIdx.x * NWAVE + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (b >= B) return;
  const int k = acc[b], y = bonus[b];
  int found = -1;
  if (k >= 0 && k <= K) {
    int lo = off[k], hi = off[k + 1];
    lo = max(lo, 0);
    hi = min(hi, Bgt);
    for (int s0 = lo; s0 < hi; s0 += 64) {
      const int sl = s0 + lane;
      const bool mt = sl < hi && keys[(int64_t)b * Bgt + sl] == y;
      const uint64_t m = __ballot(mt);
      if (m) {
        found = s0 + __builtin_ctzll(m);
        break;
      }
    }
  }
  if (lane == 0) {
    hit[b] = found >= 0;
    slot[b] = found;
  }
  for (int i = lane; i < K; i += 64)
    toks[(int64_t)b * K + i] = found >= 0 ? payload[((int64_t)b * Bgt + found) * K + i] : -1;
}

__global__ __launch_bounds__(WG) void k_cache_keys(const int32_t* topf, int ldf, const int32_t* off, int B, int K,
                                                   int Bgt, int32_t* keys) {
  const int64_t t = (int64_t)blockIdx.x * WG + threadIdx.x;
  if (t >= (int64_t)B * Bgt) return;
  const int b = (int)(t / Bgt), sl = (int)(t - (int64_t)b * Bgt);
  int val = -1;
  for (int k = 0; k <= K; ++k) {
    const int lo = off[k], hi = off[k + 1];
    if (sl >= lo && sl < hi) {
      const int i = sl - lo;
      if (i < ldf) val = topf[((int64_t)b * (K + 1) + k) * ldf + i];
      break;
    }
  }
  keys[t] = val;
}

}  // namespace ssd
