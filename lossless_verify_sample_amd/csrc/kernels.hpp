// gfx950 kernels of the verify-and-resample path.
//
// Every row of V logits is streamed from HBM once, in 2048-token blocks: a
// wave64 owns one block (32 elements per lane, 16-byte loads, consecutive
// lanes on consecutive 16-byte chunks) and reduces it with DPP to a block
// partial (block max M, sum of exp((z - M)/T)).  The workgroup that
// completes the last chunk of a row (or of a sequence, for verification)
// detects it with an agent-scope counter and runs that row's epilogue:
// merge of the partials, exact top-F by re-scanning only the blocks whose
// maxima can hold it, and the two-level Gumbel-max draw (block by ln W + g,
// then token inside the chosen block), which needs Philox for about NB + 2048
// draws per row instead of V.  Sources are cited in ssd.h.
#pragma once

#include "device.hpp"

namespace ssd {

enum Mode { M_SOFTMAX = 0, M_TOPF = 1, M_SAMPLE = 2, M_VERIFY = 3 };

constexpr int CH = 8;    // blocks per workgroup in the streaming pass (2 per wave)
constexpr int CH_R = 4;  // blocks per workgroup in the residual pass (1 per wave)

// What verification hands to the residual pass for one sequence.
struct SeqState {
  int need;   // 1: bonus from the residual at row kstar (T > 0, kstar < K)
  int kstar;
  float s;    // log2(e) / T
  float o_t;  // fl(-m_t * s): offset of target row kstar
  float o_d;  // fl(-m_d * s): offset of draft row kstar
  float kf;   // 2^(e_t - e_d) * exp(L_t - L_d): draft term scale in target units
  float m_t, m_d;
  double L_t, L_d;
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
  unsigned* cnt;            // completion counters
  ssd_row_stats* stats;     // per-row statistics out
  float* probs;             // softmax probabilities out
  int32_t* out_idx;         // top-F indices out
  float* out_val;           // top-F values out
  int32_t* tokens;          // drafted tokens out
  float* q;                 // sigma_j(x_j) out
  const int32_t* dtok;      // drafted tokens in (verification)
  const ssd_row_stats* dstats;
  const int32_t* dtopf;
  int ld_dtopf;
  int32_t* acc_len;
  int32_t* bonus;
  float* p_out;
  SeqState* state;
  float* rpart;             // residual block sums [B, NB]
  unsigned* rcnt;
};

struct Smem {
  Red red;
  int flag;
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
  int wcnt[NWAVE];
  // verification, per row j <= K
  float vm[MAX_K1];
  double vL[MAX_K1];
  int vfmb[MAX_K1];
  int vam[MAX_K1];
  int vx[MAX_K1];
  float vdm[MAX_K1];
  double vdL[MAX_K1];
  int vinS[MAX_K1];
  int vacc[MAX_K1];
};

// ---------------------------------------------------------------------------
// streaming block partial: (M, sum_x 2^(z_x*s + fl(-M*s))) for one block.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float2 block_partial(const float (&v)[32], float s) {
  float m0 = fmaxf(v[0], v[1]), m1 = fmaxf(v[2], v[3]);
#pragma unroll
  for (int k = 4; k < 32; k += 4) {
    m0 = fmaxf(m0, fmaxf(v[k], v[k + 1]));
    m1 = fmaxf(m1, fmaxf(v[k + 2], v[k + 3]));
  }
  const float M = wave_max(fmaxf(m0, m1));
  float sum = 0.f;
  if (s > 0.f) {
    const float o = (M == -INFINITY) ? 0.f : -M * s;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int k = 0; k < 32; k += 4) {
      a0 += __builtin_amdgcn_exp2f(fmaf(v[k], s, o));
      a1 += __builtin_amdgcn_exp2f(fmaf(v[k + 1], s, o));
      a2 += __builtin_amdgcn_exp2f(fmaf(v[k + 2], s, o));
      a3 += __builtin_amdgcn_exp2f(fmaf(v[k + 3], s, o));
    }
    sum = wave_sum((a0 + a1) + (a2 + a3));
  }
  return make_float2(M, sum);
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
  return min(min(sm.wcnt[0], sm.wcnt[1]), min(sm.wcnt[2], sm.wcnt[3]));
}

// Ascending compaction of {i < n : pred(i)} into out; returns the count.
template <class Pred>
__device__ int wg_compact(int n, int* out, Smem& sm, Pred pred) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int running = 0;
  for (int base = 0; base < n; base += WG) {
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
    running += sm.wcnt[0] + sm.wcnt[1] + sm.wcnt[2] + sm.wcnt[3];
  }
  __syncthreads();
  return running;
}

// Row partials -> sm.u.r.M / sm.u.r.S (all threads).
__device__ __forceinline__ void load_partials(const float2* pr, int NB, Smem& sm) {
  for (int be = threadIdx.x; be < NB; be += WG) {
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
template <int DT, bool AL>
__device__ void wg_topf(const unsigned char* rp, int64_t V, int NB, int Fsel, Smem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) sm.tau = -INFINITY;
  __syncthreads();
  if (NB > Fsel) {
    for (int be = tid; be < NB; be += WG) {
      const float mb = sm.u.r.M[be];
      int r = 0;
      for (int k = 0; k < NB; ++k) {
        const float o = sm.u.r.M[k];
        r += (o > mb) || (o == mb && k < be);
      }
      if (r == Fsel - 1) sm.tau = mb;
    }
  }
  __syncthreads();
  const float tau = sm.tau;
  const int ncb = wg_compact(NB, sm.u.r.cblk, sm, [&](int be) { return sm.u.r.M[be] >= tau; });
  if (tid == 0) sm.cnt = 0;
  __syncthreads();
  for (int c = wave; c < ncb; c += NWAVE) {
    const int be = sm.u.r.cblk[c];
    float v[32];
    load_block<DT, AL>(rp, V, be, lane, v);
    uint32_t hit = 0;
#pragma unroll
    for (int k = 0; k < 32; ++k)
      hit |= (v[k] >= tau && block_elem_index<DT>(be, lane, k) < V) ? (1u << k) : 0u;
    // few elements pass: re-read each one (cache hit) rather than index v[]
    while (hit) {
      const int k = __builtin_ctz(hit);
      hit &= hit - 1u;
      const int idx = (int)block_elem_index<DT>(be, lane, k);
      const int pos = atomicAdd(&sm.cnt, 1);
      if (pos < CAND_CAP) {
        sm.lv[pos] = load_elem<DT>(rp, idx);
        sm.li[pos] = idx;
      }
    }
  }
  __syncthreads();
  const int n = sm.cnt;
  if (n <= CAND_CAP) {
    for (int i = tid; i < n; i += WG) {
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
      for (int c = wave; c < ncb; c += NWAVE) {
        const int be = sm.u.r.cblk[c];
#pragma unroll 1
        for (int i = 0; i < 32 / VW; ++i) {
          const int e0 = be * BLK + (i * 64 + lane) * VW;
          float v[VW];
          load_chunk<DT, AL>(rp, V, e0, v);
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
  for (int be = threadIdx.x; be < NB; be += WG) {
    const double l = lnw(be);
    if (l > -INFINITY) {
      const double sc = l + (double)gumbel_of(draw1(seed, (uint32_t)be, (uint32_t)b, (uint32_t)j, st));
      best = better(best, Arg{sc, be});
    }
  }
  return wg_argmax(best, sm.red);
}

// Eight consecutive elements x0..x0+7 of a row (x0 a multiple of 8).
template <int DT, bool AL>
__device__ __forceinline__ void load8(const unsigned char* rp, int64_t V, int64_t x0, float (&o)[8]) {
  constexpr int VW = Dt<DT>::VW;
#pragma unroll
  for (int c = 0; c < 8 / VW; ++c) load_chunk<DT, AL>(rp, V, x0 + c * VW, &o[c * VW]);
}

// Token stage: argmax over x in block beta of score(z1[x], z2[x], x) + g(x);
// score returns -inf to exclude a token.  rp2 may alias rp1.
template <int DT, bool AL, class Score>
__device__ Arg token_stage(const unsigned char* rp1, const unsigned char* rp2, int64_t V, int beta,
                           uint64_t seed, int b, int j, uint32_t st, Smem& sm, Score score) {
  const int64_t x0 = (int64_t)beta * BLK + 8 * threadIdx.x;
  float z1[8], z2[8];
  load8<DT, AL>(rp1, V, x0, z1);
  load8<DT, AL>(rp2, V, x0, z2);
  Arg best{-INFINITY, (int64_t)0x7fffffff};
  if (x0 < V) {
    const uint4 wa = draws4(seed, (uint32_t)(x0 >> 2), (uint32_t)b, (uint32_t)j, st);
    const uint4 wb = draws4(seed, (uint32_t)(x0 >> 2) + 1u, (uint32_t)b, (uint32_t)j, st);
    const uint32_t w[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t x = x0 + e;
      if (x < V) {
        const double sc = score(z1[e], z2[e], (int)x);
        if (sc > -INFINITY) best = better(best, Arg{sc + (double)gumbel_of(w[e]), x});
      }
    }
  }
  return wg_argmax(best, sm.red);
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
  for (int be = threadIdx.x; be < p.NB; be += WG) lm = fmaxf(lm, sm.u.r.M[be]);
  const float m = wg_max(lm, sm.red);
  int fb = 0x7fffffff;
  double w = 0.0;
  for (int be = threadIdx.x; be < p.NB; be += WG) {
    if (sm.u.r.M[be] == m) fb = min(fb, be);
    if (!greedy) w += block_w(sm.u.r.M[be], sm.u.r.S[be], m, s);
  }
  fb = min(wg_min_i(fb, sm), p.NB - 1);  // (a NaN row matches no block)
  const double tot = wg_sum_d(w, sm.red);
  if (threadIdx.x < 64) {
    const int am = wave_first_eq<DT, AL>(rp, p.V, fb, m);
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
  wg_topf<DT, AL>(rp, p.V, p.NB, p.F, sm);
  for (int r = threadIdx.x; r < p.F; r += WG) {
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
  for (int be = threadIdx.x; be < NB; be += WG) lm = fmaxf(lm, sm.u.r.M[be]);
  const float m = wg_max(lm, sm.red);
  double w = 0.0;
  if (!greedy)
    for (int be = threadIdx.x; be < NB; be += WG) w += block_w(sm.u.r.M[be], sm.u.r.S[be], m, s);
  const double tot0 = wg_sum_d(w, sm.red);
  wg_topf<DT, AL>(rp, p.V, NB, p.F_sel, sm);
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
  for (int r = threadIdx.x; r < p.F_out; r += WG) {
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
  const Arg ts = token_stage<DT, AL>(rp, rp, p.V, beta, p.seed, b, j, ST_DRAFT_TOKEN, sm,
                                     [&](float z, float, int x) -> double {
                                       if (z == -INFINITY) return -INFINITY;
                                       return ((double)z - (double)m) * invT + (in_sblk(x, sm) ? lnC : 0.0);
                                     });
  if (threadIdx.x == 0) {
    const int x = ts.i < p.V ? (int)ts.i : 0;
    const float z = load_elem<DT>(rp, x);
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
  const double lnC = log((double)p.C);
  const int64_t r0 = (int64_t)b * K1;
  const int64_t rs = p.ld * Dt<DT>::SZ;
  // per-position draft inputs
  if (tid < K) {
    const int x = p.dtok[b * K + tid];
    const ssd_row_stats ds = p.dstats[r0 + tid];
    int inS = 0;
    for (int f = 0; f < p.F; ++f) inS |= (p.dtopf[(r0 + tid) * p.ld_dtopf + f] == x);
    sm.vx[tid] = x;
    sm.vdm[tid] = ds.max;
    sm.vdL[tid] = ds.lse;
    sm.vinS[tid] = inS;
  }
  // merge the partials of rows 0..K, several rows per staging round
  const int rpg = max(1, STAGE / NB);
  for (int g0 = 0; g0 < K1; g0 += rpg) {
    const int n = min(rpg, K1 - g0);
    __syncthreads();
    const float2* src = p.part + (r0 + g0) * NB;
    for (int i = tid; i < n * NB; i += WG) sm.u.stage[i] = src[i];
    __syncthreads();
    for (int jj = wave; jj < n; jj += NWAVE) {
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
      }
    }
  }
  __syncthreads();
  // argmax of every row (greedy decisions, statistics)
  const bool need_am = greedy || p.stats != nullptr;
  if (need_am)
    for (int j = wave; j < K1; j += NWAVE) {
      const int am = wave_first_eq<DT, AL>(p.x + (r0 + j) * rs, p.V, sm.vfmb[j], sm.vm[j]);
      if (lane == 0) sm.vam[j] = am;
    }
  __syncthreads();
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
        const float zt = load_elem<DT>(p.x + (r0 + j) * rs, x);
        const float zd = load_elem<DT>(p.xd + (r0 + j) * rs, x);
        const double lp = ((double)zt - (double)sm.vm[j]) * invT - sm.vL[j];
        const double ls = ((double)zd - (double)sm.vdm[j]) * invT + (sm.vinS[j] ? lnC : 0.0) - sm.vdL[j];
        pj = exp(lp);
        const double rho = (zd == -INFINITY) ? (zt == -INFINITY ? 0.0 : INFINITY) : exp(lp - ls);
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
      const float mt = sm.vm[ks], md = sm.vdm[ks];
      ss.need = 1;
      ss.kstar = ks;
      ss.s = s;
      ss.o_t = -mt * s;
      ss.o_d = -md * s;
      const double et = (double)ss.o_t + (double)mt * (double)s;
      const double ed = (double)ss.o_d + (double)md * (double)s;
      ss.kf = (float)(exp2(et - ed) * exp(sm.vL[ks] - sm.vdL[ks]));
      ss.m_t = mt;
      ss.m_d = md;
      ss.L_t = sm.vL[ks];
      ss.L_d = sm.vdL[ks];
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
  const Arg ts = token_stage<DT, AL>(rp, rp, p.V, bs.i < NB ? (int)bs.i : 0, p.seed, b, K, ST_BONUS_TOKEN, sm,
                                     [&](float z, float, int) -> double {
                                       return z == -INFINITY ? -INFINITY : ((double)z - (double)m) * invT;
                                     });
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
  for (int be = threadIdx.x; be < NB; be += WG) sm.u.r.S[be] = p.rpart[(int64_t)b * NB + be];
  if (threadIdx.x < p.F) sm.tidx[threadIdx.x] = p.dtopf[row * p.ld_dtopf + threadIdx.x];
  __syncthreads();
  double w = 0.0;
  for (int be = threadIdx.x; be < NB; be += WG) w += (double)sm.u.r.S[be];
  const double tot = wg_sum_d(w, sm.red);
  const bool res = tot > 0.0;
  if (!res) load_partials(p.part + row * NB, NB, sm);  // no residual mass: sample p_k*
  const float mt = ss.m_t, md = ss.m_d, s = ss.s;
  const double Lt = ss.L_t, Ld = ss.L_d;
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
    const Arg tp = token_stage<DT, AL>(rt, rt, p.V, beta, p.seed, b, ks, ST_BONUS_TOKEN, sm,
                                       [&](float zt, float, int) -> double {
                                         return zt == -INFINITY ? -INFINITY : ((double)zt - (double)mt) * invT;
                                       });
    bonus = (int)tp.i;
  }
  if (threadIdx.x == 0) p.bonus[b] = (bonus >= 0 && bonus < p.V) ? bonus : 0;
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------
// Release this workgroup's partial stores and count it in; true in every
// thread of the workgroup that completes the group.
__device__ __forceinline__ bool arrive_last(unsigned* ctr, unsigned total, Smem& sm) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(ctr, 1u);
    sm.flag = (prev == total - 1u);
  }
  __syncthreads();
  if (!sm.flag) return false;
  __threadfence();
  if (threadIdx.x == 0) *ctr = 0u;  // leave the counter cleared for the next call
  return true;
}

template <int DT, bool AL, int MODE>
__global__ __launch_bounds__(WG, 6) void k_stream(Params p) {
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
  const int b0 = chunk * CH + wave, b1 = b0 + NWAVE;
  float v0[32], v1[32];
  const bool h0 = b0 < p.NB, h1 = b1 < p.NB;
  if (h0) load_block<DT, AL>(rp, p.V, b0, lane, v0);
  if (h1) load_block<DT, AL>(rp, p.V, b1, lane, v1);
  if (h0) {
    const float2 r = block_partial(v0, s);
    if (lane == 0) p.part[row * p.NB + b0] = r;
  }
  if (h1) {
    const float2 r = block_partial(v1, s);
    if (lane == 0) p.part[row * p.NB + b1] = r;
  }
  if constexpr (MODE == M_VERIFY) {
    const int b = (int)(row / K1);
    if (!arrive_last(p.cnt + b, (unsigned)(K1 * p.nchunk), sm)) return;
    epi_verify<DT, AL>(p, b, sm);
  } else {
    if (!arrive_last(p.cnt + row, (unsigned)p.nchunk, sm)) return;
    if constexpr (MODE == M_SOFTMAX) epi_softmax<DT, AL>(p, row, sm);
    if constexpr (MODE == M_TOPF) epi_topf<DT, AL>(p, row, sm);
    if constexpr (MODE == M_SAMPLE) epi_sample<DT, AL>(p, row, sm);
  }
}

// Residual pass for sequences rejected at k* < K: block sums of
// max(0, p - sigma) over target row k* and draft row k*, in the target's
// units scaled by exp(L_t) 2^(e_t) (a constant per sequence).
template <int DT, bool AL>
__global__ __launch_bounds__(WG) void k_residual(Params p) {
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
  __syncthreads();
  const int be = chunk * CH_R + wave;
  if (be < p.NB) {
    float vt[32], vd[32];
    load_block<DT, AL>(rt, p.V, be, lane, vt);
    load_block<DT, AL>(rd, p.V, be, lane, vd);
    const float s = ss.s, ot = ss.o_t, od = ss.o_d, nk = -ss.kf;
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
  if (!arrive_last(p.rcnt + b, (unsigned)p.nchunk, sm)) return;
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
