// gfx950 kernels of the verify-and-resample path.
//
// Every row of V logits is streamed from HBM once, in 2048-token blocks: a
// wave64 owns one block (32 elements per lane, 16-byte loads, consecutive
// lanes on consecutive 16-byte chunks) and reduces it with DPP to a block
// partial (block max M and the sum of exp((z - M)/T), or the block argmax for
// greedy rows).  A second kernel then runs one workgroup of four waves per
// row (or per sequence, for verification) over those partials: merge, exact
// top-F, and the two-level draw (a block by its weight, then a token inside
// the chosen block, which is re-read), so Philox runs for about NB + 2048
// draws per row instead of V.  The kernel boundary between the two makes the
// partials visible without any cross-workgroup synchronisation.
//
// Both levels of the draw use the exponential-race form of the Gumbel-max
// trick: argmax_x ln w_x + g_x with g_x = -ln(-ln u_x) is the same choice as
// argmin_x (-ln u_x) / w_x, which needs one hardware log2 and one exp2 (or a
// reciprocal) per candidate and no second logarithm.  Keys are compared as
// (float key, index) pairs packed in 64 bits, ties going to the lower index.
// Sources are cited in ssd.h.
#pragma once

#include "device.hpp"

namespace ssd {

enum Mode { M_SOFTMAX = 0, M_TOPF = 1, M_SAMPLE = 2, M_VERIFY = 3 };

constexpr int CH = 8;             // blocks per workgroup in the streaming pass (2 per wave)
constexpr int CH_R = 4;           // blocks per workgroup in the residual pass (1 per wave)
constexpr int TPT = BLK / EWG;    // tokens per epilogue thread in a token stage
constexpr int NBT = MAX_NB / EWG; // blocks per epilogue thread
static_assert(TPT == 8 && NBT == 2, "epilogue layout assumes 256 threads over 2048-token blocks");

// What verification hands to the residual pass for one sequence.
struct SeqState {
  int need;      // 1: bonus from the residual at row kstar (T > 0, kstar < K)
  int kstar;
  float s;       // log2(e) / T
  float o_t;     // fl(-m_t s): offset of target row kstar in the residual pass
  float o_d;     // fl(-m_d s): the same for draft row kstar
  float kf;      // draft term in the target's units: 2^(eps_t - eps_d) exp(L_t - L_d)
  float m_t;     // max of target row kstar
  float pad;
  double invT;   // 1 / T
  double D0;     // (m_t - m_d) / T + L_t - L_d
  double lnC;
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
  float4* part;             // block partials [rows, NB]: (M, S, I, M2)
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

// LDS of an epilogue workgroup.
struct ESm {
  float rf[2][ENW];         // reduction slots, one per call site
  double rd[2][ENW];
  uint64_t ru[6][ENW];
  int ri[2][ENW];
  float M[MAX_NB];          // block maxima of the row
  float M2[MAX_NB];         // second values of the blocks
  int I[MAX_NB];            // argmax indices of the blocks
  float S[MAX_NB];          // block sums (verification: row K)
  int cblk[MAX_NB];         // candidate blocks for top-F
  uint64_t cand[CAND_CAP];  // top-F candidates as (value desc, index asc) keys
  int nre;                  // candidates appended by block re-reads
  int ks;
  float tval[MAX_F];        // top-F result, sorted
  int tidx[MAX_F];
  float es[MAX_F];          // 2^((z_f - m) s) of the top-F set
  float vm[MAX_K1];         // verification, per row j <= K
  double vL[MAX_K1];
  int vfb[MAX_K1];
  int vam[MAX_K1];
};

// ---------------------------------------------------------------------------
// streaming block partial of one block (one wave): P = (M, S, I, M2) with M
// the block maximum; S = sum_x 2^(z_x*s + fl(-M*s)) for T > 0 (else 0); I
// the lowest index holding M (as int bits, -1 when not wanted); M2 the
// largest value left after removing that element, i.e. the second-largest
// value counted with multiplicity (M when not wanted).  A lane holds its 32
// elements as NG groups of VW (one 16-byte chunk each): element e of group g
// of lane l is index beta*BLK + (g*64 + l)*VW + e.
// ---------------------------------------------------------------------------
template <int VW>
__device__ __forceinline__ float group_max(const float* x) {
  if constexpr (VW == 8) return fmax3(fmax3(x[0], x[1], x[2]), fmax3(x[3], x[4], x[5]), fmax3(x[6], x[7], x[7]));
  else return fmax3(fmax3(x[0], x[1], x[2]), x[3], x[3]);
}
template <int NG>
__device__ __forceinline__ float lane_max(const float* g) {
  if constexpr (NG == 4) return fmax3(fmax3(g[0], g[1], g[2]), g[3], g[3]);
  else return fmax3(fmax3(g[0], g[1], g[2]), fmax3(g[3], g[4], g[5]), fmax3(g[6], g[7], g[7]));
}

// I and (when WM2) M2 of a block from its group maxima g and lane maxima lm:
// the first group (in index order) with a lane holding M, its lowest such
// lane L and lowest element e.  M2: if M occurs twice it is M; otherwise the
// maximum over the other lanes and over lane L's values other than M.  Every
// register access is static (one uniform branch per group), which keeps the
// element arrays out of scratch memory.
template <int DT, bool WM2>
__device__ __forceinline__ void block_top(const float (&v)[32], const float* g, float lm, int beta, int lane,
                                          float4& P) {
  constexpr int VW = Dt<DT>::VW, NG = 32 / VW;
  const float M = P.x;
  int gi = -1;
  uint64_t bal = 0;
#pragma unroll
  for (int i = NG - 1; i >= 0; --i) {
    const uint64_t bi = __ballot(g[i] == M);
    if (bi) {
      gi = i;
      bal = bi;
    }
  }
  if (gi < 0) return;  // (a NaN maximum)
  const int L = (int)__builtin_ctzll(bal);
  int es = 0;
  float o = -INFINITY;
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    if (gi == i) {
      int cnt = 0;
#pragma unroll
      for (int e = VW - 1; e >= 0; --e) {
        if ((__ballot(v[i * VW + e] == M) >> L) & 1ull) {
          es = e;
          ++cnt;
        }
      }
      if constexpr (WM2) {
        float y[VW], gg[NG];
#pragma unroll
        for (int e = 0; e < VW; ++e) y[e] = (v[i * VW + e] == M) ? -INFINITY : v[i * VW + e];
#pragma unroll
        for (int k = 0; k < NG; ++k) gg[k] = (k == i) ? -INFINITY : g[k];
        o = fmax3(cnt > 1 ? M : group_max<VW>(y), lane_max<NG>(gg), lane_max<NG>(gg));
      }
    }
  }
  P.z = __int_as_float(beta * BLK + (gi * 64 + L) * VW + es);
  if constexpr (WM2) P.w = wave_max3(lane == L ? o : lm);
}

template <int DT, int MODE>
__device__ __forceinline__ float4 block_partial(const float (&v)[32], float s, int beta, int lane) {
  constexpr int VW = Dt<DT>::VW, NG = 32 / VW;
  // every mode but top-F sums; verification needs I only for greedy rows; only
  // sampling and top-F select by value and need M2
  constexpr bool WS = MODE != M_TOPF, WM2 = MODE == M_SAMPLE || MODE == M_TOPF;
  float g[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) g[i] = group_max<VW>(&v[i * VW]);
  const float lm = lane_max<NG>(g);
  float4 P = make_float4(wave_max3(lm), 0.f, __int_as_float(-1), 0.f);
  P.w = P.x;
  if (WS && s > 0.f) {
    const float o = (P.x == -INFINITY) ? 0.f : -P.x * s;
    float a0 = __builtin_amdgcn_exp2f(fmaf(v[0], s, o)), a1 = __builtin_amdgcn_exp2f(fmaf(v[1], s, o));
    float a2 = __builtin_amdgcn_exp2f(fmaf(v[2], s, o)), a3 = __builtin_amdgcn_exp2f(fmaf(v[3], s, o));
#pragma unroll
    for (int k = 4; k < 32; k += 4) {
      a0 += __builtin_amdgcn_exp2f(fmaf(v[k], s, o));
      a1 += __builtin_amdgcn_exp2f(fmaf(v[k + 1], s, o));
      a2 += __builtin_amdgcn_exp2f(fmaf(v[k + 2], s, o));
      a3 += __builtin_amdgcn_exp2f(fmaf(v[k + 3], s, o));
    }
    P.y = wave_sum((a0 + a1) + (a2 + a3));
  }
  if (MODE != M_VERIFY || !(s > 0.f)) block_top<DT, WM2>(v, g, lm, beta, lane, P);
  return P;
}

// Exponent x (base 2) of block weight W = S * 2^x relative to row max m:
// undoes the rounding of the block offset fl(-M*s) used while streaming.
__device__ __forceinline__ double block_x(float M, float m, float s) {
  const float o = -M * s;
  const double e = (double)o + (double)M * (double)s;
  return ((double)M - (double)m) * (double)s - e;
}
// W relative to the row maximum (0 for empty blocks).
__device__ __forceinline__ float block_w(float M, float S, float m, float s) {
  if (M == -INFINITY || !(S > 0.f)) return 0.f;
  return S * __builtin_amdgcn_exp2f((float)block_x(M, m, s));
}

// ---------------------------------------------------------------------------
// epilogue building blocks (EWG threads; thread t owns blocks t + k*EWG)
// ---------------------------------------------------------------------------
// Partials of one row: (M, S) of this thread's blocks into registers, M, M2
// and I of every block into LDS; also clears the top-F re-read counter.  The
// caller passes a barrier before LDS is read.
__device__ __forceinline__ void load_row_partials(const float4* pr, int NB, ESm& sm, float (&M)[NBT],
                                                  float (&S)[NBT]) {
  if (threadIdx.x == 0) sm.nre = 0;
#pragma unroll
  for (int k = 0; k < NBT; ++k) {
    const int be = threadIdx.x + k * EWG;
    const float4 v = be < NB ? pr[be] : make_float4(-INFINITY, 0.f, 0.f, -INFINITY);
    M[k] = v.x;
    S[k] = v.y;
    if (be < NB) {
      sm.M[be] = v.x;
      sm.M2[be] = v.w;
      sm.I[be] = __float_as_int(v.z);
    }
  }
}

// Lowest index of value m inside block beta (one wave).
template <int DT, bool AL>
__device__ __forceinline__ int wave_first_eq(const unsigned char* rp, int64_t V, int beta, float m) {
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

// Exact top-Fs of a row into sm.tval / sm.tidx (value desc, index asc).  The
// Fs-th largest block maximum tau bounds the Fs-th largest element from
// below, so every top element lies in a candidate block (maximum >= tau).  A
// candidate whose second value is below tau holds exactly one element >= tau,
// its maximum, whose index the partial carries; only the other candidates are
// re-read, and only their elements >= tau are ranked.  Every wave finds tau
// itself (a 32-step radix search on ballots over the order-preserving keys of
// the block maxima), so no barrier precedes the re-reads.  Needs
// load_row_partials and a barrier since; ends with a barrier.
template <int DT, bool AL>
__device__ __forceinline__ void row_topf(const unsigned char* rp, int V, int NB, int Fs, ESm& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int PL = MAX_NB / 64;
  const int npl = (NB + 63) >> 6;
  uint32_t key[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int be = lane + 64 * i;
    key[i] = (i < npl && be < NB) ? ord_key(sm.M[be]) : 0u;
  }
  // tau: the largest key c with at least Fs block maxima at or above it
  uint32_t tk = 0;
  if (NB > Fs) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = tk | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < PL; ++i)
        if (i < npl) cnt += __popcll(__ballot(key[i] >= c));
      if (cnt >= Fs) tk = c;
    }
  }
  const float tau = NB > Fs ? ord_val(tk) : -INFINITY;
  uint64_t cmk[PL], rmk[PL];
  int n1 = 0;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int be = lane + 64 * i;
    const bool c = i < npl && be < NB && key[i] >= tk;
    cmk[i] = __ballot(c);
    rmk[i] = __ballot(c && (NB <= Fs || sm.M2[be] >= tau));
    n1 += __popcll(cmk[i] & ~rmk[i]);
  }
  // wave 0 lists the candidate blocks and the one-element candidates
  const uint64_t below = (1ull << lane) - 1ull;
  if (wave == 0) {
    int nc = 0, k1 = 0;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int be = lane + 64 * i;
      const uint64_t one = cmk[i] & ~rmk[i];
      if ((cmk[i] >> lane) & 1ull) sm.cblk[nc + __popcll(cmk[i] & below)] = be;
      if (((one >> lane) & 1ull) && k1 + __popcll(one & below) < CAND_CAP)
        sm.cand[k1 + __popcll(one & below)] = vi_key(sm.M[be], sm.I[be]);
      nc += __popcll(cmk[i]);
      k1 += __popcll(one);
    }
  }
  // the other candidates are re-read, round-robin over the waves
  int nr = 0;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    uint64_t rr = rmk[i];
    while (rr) {
      const int be = 64 * i + (int)__builtin_ctzll(rr);
      rr &= rr - 1ull;
      if (nr++ % ENW != wave) continue;
      float v[32];
      if ((be + 1) * BLK <= V) load_block_full<DT, AL>(rp, be, lane, v);
      else load_block<DT, AL>(rp, V, be, lane, v);
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const int idx = block_elem_index<DT>(be, lane, k);
        if (v[k] >= tau && idx < V) {
          const int pos = n1 + atomicAdd(&sm.nre, 1);
          if (pos < CAND_CAP) sm.cand[pos] = vi_key(v[k], idx);
        }
      }
    }
  }
  int nc = 0;
#pragma unroll
  for (int i = 0; i < PL; ++i) nc += __popcll(cmk[i]);
  __syncthreads();
  const int n = n1 + sm.nre;
  if (n <= CAND_CAP) {
    for (int i = tid; i < n; i += EWG) {
      const uint64_t ki = sm.cand[i];
      int r = 0;
      for (int c = 0; c < n; ++c) r += sm.cand[c] > ki;
      if (r < Fs) {
        sm.tval[r] = key_val(ki);
        sm.tidx[r] = (int)key_idx(ki);
      }
    }
  } else {
    // Many ties at the threshold: take the best key below the previous one,
    // Fs times, over the candidate blocks (alternating reduction slots).
    uint64_t prev = ~0ull;
    constexpr int VW = Dt<DT>::VW;
    for (int r = 0; r < Fs; ++r) {
      uint64_t best = 0;
      for (int c = wave; c < nc; c += ENW) {
        const int be = sm.cblk[c];
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
      best = wg_max_u64(best, sm.ru[4 + (r & 1)]);
      if (tid == 0) {
        sm.tval[r] = key_val(best);
        sm.tidx[r] = (int)key_idx(best);
      }
      prev = best;
    }
  }
  __syncthreads();
}

// Block stage of the two-level draw: argmin over blocks of -log2(u_be) / W_be
// (the common factor ln 2 dropped); wfn(be, k) gives W_be >= 0 for the k-th
// block of this thread.  Returns the chosen block, -1 if no block has mass.
template <class WF>
__device__ int block_stage(int NB, uint64_t seed, int b, int j, uint32_t st, uint64_t* slot, WF wfn) {
  uint64_t best = NO_KEY;
#pragma unroll
  for (int k = 0; k < NBT; ++k) {
    const int be = threadIdx.x + k * EWG;
    if (be < NB) {
      const float W = wfn(be, k);
      if (W > 0.f) {
        const float key = neg_log2_u(draw1(seed, (uint32_t)be, (uint32_t)b, (uint32_t)j, st)) *
                          __builtin_amdgcn_rcpf(W);
        best = umin64(best, race_key(key, be));
      }
    }
  }
  best = wg_min_u64(best, slot);
  return best == NO_KEY ? -1 : (int)(uint32_t)best;
}

// TPT consecutive elements x0.. of a row; past V reads as -inf.
template <int DT, bool AL>
__device__ __forceinline__ void load_run(const unsigned char* rp, int V, int x0, float (&z)[TPT]) {
  if constexpr (AL) {
    if (x0 + TPT <= V) {
      const uint4* a = reinterpret_cast<const uint4*>(rp + (size_t)x0 * Dt<DT>::SZ);
      if constexpr (DT == SSD_F32) {
        decode16<DT>(a[0], &z[0]);
        decode16<DT>(a[1], &z[4]);
      } else {
        decode16<DT>(a[0], z);
      }
      return;
    }
  }
#pragma unroll
  for (int e = 0; e < TPT; ++e) {
    const bool in = x0 + e < V;
    const float x = load_elem<DT>(rp, in ? x0 + e : 0);
    z[e] = in ? x : -INFINITY;
  }
}

// Token stage of the two-level draw over a block: thread t holds tokens
// x0 .. x0 + TPT - 1 (x0 = beta*BLK + TPT*t) with their Philox words; tfn(e)
// gives the log2 of the inverse weight of token x0 + e up to a constant
// common to the block (+inf excludes it).  Returns the winner (-1 if none).
template <class TF>
__device__ int token_race(int x0, int V, uint64_t seed, int b, int j, uint32_t st, uint64_t* slot, TF tfn) {
  const uint4 wa = draws4(seed, (uint32_t)(x0 >> 2), (uint32_t)b, (uint32_t)j, st);
  const uint4 wb = draws4(seed, (uint32_t)(x0 >> 2) + 1u, (uint32_t)b, (uint32_t)j, st);
  const uint32_t w[TPT] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
  uint64_t best = NO_KEY;
#pragma unroll
  for (int e = 0; e < TPT; ++e) {
    const float t = tfn(e);
    if (x0 + e < V && t < INFINITY) {
      const float key = neg_log2_u(w[e]) * __builtin_amdgcn_exp2f(t);
      best = umin64(best, race_key(key, x0 + e));
    }
  }
  best = wg_min_u64(best, slot);
  return best == NO_KEY ? -1 : (int)(uint32_t)best;
}

// Bit e set when token x0 + e is one of idx[0 .. F).
__device__ __forceinline__ uint32_t set_mask(const int* idx, int F, int x0) {
  uint32_t msk = 0;
  for (int f = 0; f < F; ++f) {
    const uint32_t d = (uint32_t)(idx[f] - x0);
    if (d < (uint32_t)TPT) msk |= 1u << d;
  }
  return msk;
}

// ---------------------------------------------------------------------------
// epilogues
// ---------------------------------------------------------------------------
template <int DT, bool AL>
__device__ void epi_softmax(const Params& p, int64_t row, ESm& sm) {
  const int tid = threadIdx.x;
  const float T = p.temp[row];
  const bool greedy = !(T > 0.f);
  const float s = greedy ? 0.f : (float)(LOG2E / (double)T);
  const int NB = p.NB;
  const unsigned char* rp = p.x + row * p.ld * Dt<DT>::SZ;
  float M[NBT], S[NBT];
  load_row_partials(p.part + row * NB, NB, sm, M, S);
  const float m = wg_max(fmaxf(M[0], M[1]), sm.rf[0]);
  int fb = 0x7fffffff;
  double w = 0.0;
#pragma unroll
  for (int k = 0; k < NBT; ++k) {
    const int be = tid + k * EWG;
    if (be < NB && M[k] == m) fb = min(fb, be);
    if (!greedy) w += (double)block_w(M[k], S[k], m, s);
  }
  fb = min(wg_min_i(fb, sm.ri[0]), NB - 1);  // (a NaN row matches no block)
  const double tot = greedy ? 1.0 : wg_sum_d(w, sm.rd[0]);
  if (tid == 0) {
    ssd_row_stats st;
    st.lse = greedy ? 0.0 : log(tot);
    st.max = m;
    st.argmax = sm.I[fb];  // the partials carry each block's argmax
    p.stats[row] = st;
  }
  (void)rp;
}

template <int DT, bool AL>
__device__ void epi_topf(const Params& p, int64_t row, ESm& sm) {
  const unsigned char* rp = p.x + row * p.ld * Dt<DT>::SZ;
  float M[NBT], S[NBT];
  load_row_partials(p.part + row * p.NB, p.NB, sm, M, S);
  __syncthreads();
  row_topf<DT, AL>(rp, (int)p.V, p.NB, p.F, sm);
  for (int r = threadIdx.x; r < p.F; r += EWG) {
    p.out_idx[row * p.F + r] = sm.tidx[r];
    if (p.out_val) p.out_val[row * p.F + r] = sm.tval[r];
  }
}

template <int DT, bool AL>
__device__ void epi_sample(const Params& p, int64_t row, ESm& sm) {
  const int tid = threadIdx.x;
  const int K1 = p.K + 1;
  const int b = (int)(row / K1), j = (int)(row % K1);
  const float T = p.temp[b];
  const bool greedy = !(T > 0.f);
  const float s = greedy ? 0.f : (float)(LOG2E / (double)T);
  const int NB = p.NB, V = (int)p.V, F = p.F;
  const float C = p.C;
  const unsigned char* rp = p.x + row * p.ld * Dt<DT>::SZ;
  float M[NBT], S[NBT];
  load_row_partials(p.part + row * NB, NB, sm, M, S);
  const float m = wg_max(fmaxf(M[0], M[1]), sm.rf[0]);
  float w[NBT];
  double wsum = 0.0;
#pragma unroll
  for (int k = 0; k < NBT; ++k) {
    w[k] = greedy ? 0.f : block_w(M[k], S[k], m, s);
    wsum += (double)w[k];
  }
  const double tot0 = greedy ? 1.0 : wg_sum_d(wsum, sm.rd[0]);
  row_topf<DT, AL>(rp, V, NB, p.F_sel, sm);
  // sigma_{F,C}: the first F of the top list form S; their weights
  if (!greedy && tid < F) sm.es[tid] = __builtin_amdgcn_exp2f((sm.tval[tid] - m) * s);
  __syncthreads();
  auto row_lse = [&]() -> double {  // ln of the sigma normaliser, relative to m
    double zs = 0.0;
    for (int f = 0; f < F; ++f) zs += (double)sm.es[f];
    return log((tot0 - zs) + (double)C * zs);
  };
  if (tid == 0) {
    ssd_row_stats st;
    st.lse = greedy ? 0.0 : row_lse();
    st.max = m;
    st.argmax = sm.tidx[0];
    p.stats[row] = st;
  }
  for (int r = tid; r < p.F_out; r += EWG) {
    if (p.out_idx) p.out_idx[row * p.F_out + r] = sm.tidx[r];
    if (p.out_val) p.out_val[row * p.F_out + r] = sm.tval[r];
  }
  if (j == p.K) return;  // row K only predicts the bonus after K acceptances
  if (greedy) {
    if (tid == 0) {
      p.tokens[b * p.K + j] = sm.tidx[0];
      p.q[b * p.K + j] = 1.0f;
    }
    return;
  }
  int beta = block_stage(NB, p.seed, b, j, ST_DRAFT_BLOCK, sm.ru[0], [&](int be, int k) -> float {
    float corr = 0.f;
    for (int f = 0; f < F; ++f)
      if (sm.tidx[f] / BLK == be) corr += sm.es[f];
    return corr > 0.f ? fmaxf(w[k] - corr, 0.f) + C * corr : w[k];
  });
  if (beta < 0) beta = 0;  // no block of mass only for invalid rows
  const int x0 = beta * BLK + TPT * tid;
  float z[TPT];
  load_run<DT, AL>(rp, V, x0, z);
  const uint32_t smask = set_mask(sm.tidx, F, x0);
  const float nc2 = -__builtin_amdgcn_logf(C);  // -log2 C >= 0
  const float Mb = sm.M[beta];
  const int x = token_race(x0, V, p.seed, b, j, ST_DRAFT_TOKEN, sm.ru[1], [&](int e) -> float {
    if (!(z[e] > -INFINITY)) return INFINITY;
    return (Mb - z[e]) * s + (((smask >> e) & 1u) ? nc2 : 0.f);
  });
  const uint32_t d = (uint32_t)(x - x0);
  if (x >= 0 && d < (uint32_t)TPT) {
    // the owner of the winning token writes it with sigma_j(x)
    float zx = z[0];
#pragma unroll
    for (int e = 1; e < TPT; ++e) zx = (d == (uint32_t)e) ? z[e] : zx;
    const bool inS = (smask >> d) & 1u;
    const double lq = ((double)zx - (double)m) * (1.0 / (double)T) + (inS ? log((double)C) : 0.0) - row_lse();
    p.tokens[b * p.K + j] = x;
    p.q[b * p.K + j] = (float)exp(lq);
  } else if (x < 0 && tid == 0) {
    p.tokens[b * p.K + j] = 0;
    p.q[b * p.K + j] = 0.f;
  }
}

template <int DT, bool AL>
__device__ void epi_verify(const Params& p, int b, ESm& sm) {
  const int K = p.K, K1 = K + 1, NB = p.NB, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int V = (int)p.V;
  const float T = p.temp[b];
  const bool greedy = !(T > 0.f);
  const float s = greedy ? 0.f : (float)(LOG2E / (double)T);
  const double invT = greedy ? 0.0 : 1.0 / (double)T;
  const int64_t r0 = (int64_t)b * K1;
  const int64_t rs = p.ld * Dt<DT>::SZ;
  // wave 0, lane j < K: drafted token, sigma_j(x_j), the target logit at x_j
  // captured by the streaming pass; lane j <= K: the draft row statistics
  int xj = -1;
  float qj = 0.f, ztj = 0.f, dmax = 0.f;
  double dlse = 0.0;
  if (tid < K) {
    xj = p.dtok[b * K + tid];
    qj = p.dq[b * K + tid];
    ztj = p.zcap[b * K + tid];
  }
  if (tid <= K && !greedy) {
    const ssd_row_stats ds = p.dstats[r0 + tid];
    dmax = ds.max;
    dlse = ds.lse;
  }
  // row statistics: wave w merges rows j = w, w + ENW, ...
  constexpr int PL = MAX_NB / 64;
  for (int j = wave; j < K1; j += ENW) {
    const float4* pr = p.part + (r0 + j) * NB;
    float Mv[PL], Sv[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int be = lane + 64 * i;
      const float4 v = be < NB ? pr[be] : make_float4(-INFINITY, 0.f, 0.f, 0.f);
      Mv[i] = v.x;
      Sv[i] = v.y;
    }
    float lm = Mv[0];
#pragma unroll
    for (int i = 1; i < PL; ++i) lm = fmaxf(lm, Mv[i]);
    const float m = wave_max(lm);
    int fb = 0x7fffffff;
    double wsum = 0.0;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      if (Mv[i] == m) fb = min(fb, lane + 64 * i);
      if (!greedy) wsum += (double)block_w(Mv[i], Sv[i], m, s);
    }
    fb = min(wave_min_i(fb), NB - 1);
    wsum = wave_sum_d(wsum);
    if (j == K) {
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int be = lane + 64 * i;
        if (be < NB) {
          sm.M[be] = Mv[i];
          sm.S[be] = Sv[i];
        }
      }
    }
    if (lane == 0) {
      sm.vm[j] = m;
      sm.vL[j] = greedy ? 0.0 : log(wsum);
      sm.vfb[j] = fb;
      // greedy rows carry the block argmax in their partial
      sm.vam[j] = greedy ? __float_as_int(pr[fb].z) : -1;
    }
  }
  __syncthreads();
  // argmax of the T > 0 rows is only needed for the optional statistics
  if (!greedy && p.stats) {
    for (int j = wave; j < K1; j += ENW) {
      const int am = wave_first_eq<DT, AL>(p.x + (r0 + j) * rs, V, sm.vfb[j], sm.vm[j]);
      if (lane == 0) sm.vam[j] = am;
    }
    __syncthreads();
  }
  // acceptance decisions (wave 0, lane j < K) and p_j(x_j) for every position
  if (wave == 0) {
    bool acc = false;
    if (lane < K) {
      double pj = 0.0;
      if (xj >= 0 && xj < V) {
        if (greedy) {
          acc = (xj == sm.vam[lane]);
          pj = acc ? 1.0 : 0.0;
        } else {
          pj = exp(((double)ztj - (double)sm.vm[lane]) * invT - sm.vL[lane]);
          const double q = (double)qj;
          const double rho = q > 0.0 ? pj / q : (pj > 0.0 ? INFINITY : 0.0);
          const float u = uniform_of(draw1(p.seed, 0u, (uint32_t)b, (uint32_t)lane, ST_ACCEPT));
          acc = (double)u < rho;
        }
      }
      p.p_out[b * K + lane] = (float)pj;
    }
    const uint64_t rej = __ballot(lane < K && !acc);
    const int ks = rej ? (int)__builtin_ctzll(rej) : K;
    SeqState ss{};
    if (!greedy && ks < K) {
      // hand-over to the residual pass (values of target and draft row k*)
      const float mt = sm.vm[ks];
      const float md = rl_f(dmax, ks);
      const double Ld = rl_d(dlse, ks), Lt = sm.vL[ks];
      ss.need = 1;
      ss.kstar = ks;
      ss.s = s;
      ss.m_t = mt;
      ss.o_t = -mt * s;
      ss.o_d = -md * s;
      const double et = (double)ss.o_t + (double)mt * (double)s;
      const double ed = (double)ss.o_d + (double)md * (double)s;
      ss.invT = invT;
      ss.D0 = ((double)mt - (double)md) * invT + Lt - Ld;
      ss.lnC = log((double)p.C);
      ss.kf = (float)(exp2(et - ed) * exp(Lt - Ld));
    }
    if (lane == 0) {
      sm.ks = ks;
      p.acc_len[b] = ks;
      p.state[b] = ss;
      if (greedy) p.bonus[b] = sm.vam[ks];
    }
  }
  if (p.stats && tid < K1) {
    ssd_row_stats st;
    st.lse = sm.vL[tid];
    st.max = sm.vm[tid];
    st.argmax = sm.vam[tid];
    p.stats[r0 + tid] = st;
  }
  if (greedy) return;
  __syncthreads();
  if (sm.ks < K) return;
  // all K accepted: bonus ~ p_K (row K's partials are in sm.M / sm.S)
  const float m = sm.vm[K];
  int beta = block_stage(NB, p.seed, b, K, ST_BONUS_BLOCK, sm.ru[0], [&](int be, int) -> float {
    return block_w(sm.M[be], sm.S[be], m, s);
  });
  if (beta < 0) beta = 0;
  const unsigned char* rp = p.x + (r0 + K) * rs;
  const int x0 = beta * BLK + TPT * tid;
  float z[TPT];
  load_run<DT, AL>(rp, V, x0, z);
  const float Mb = sm.M[beta];
  const int x = token_race(x0, V, p.seed, b, K, ST_BONUS_TOKEN, sm.ru[1], [&](int e) -> float {
    return z[e] > -INFINITY ? (Mb - z[e]) * s : INFINITY;
  });
  if (tid == 0) p.bonus[b] = x >= 0 ? x : 0;
}

template <int DT, bool AL>
__device__ void epi_residual(const Params& p, int b, const SeqState& ss, ESm& sm) {
  const int tid = threadIdx.x, K1 = p.K + 1, NB = p.NB, ks = ss.kstar, V = (int)p.V, F = p.F;
  const int64_t row = (int64_t)b * K1 + ks;
  const int64_t rs = p.ld * Dt<DT>::SZ;
  const unsigned char* rt = p.x + row * rs;
  const unsigned char* rd = p.xd + row * rs;
  const float s = ss.s, mt = ss.m_t;
  // residual block sums; target row k*'s partials for the no-residual case
  float R[NBT], M[NBT], S[NBT];
  load_row_partials(p.part + row * NB, NB, sm, M, S);
#pragma unroll
  for (int k = 0; k < NBT; ++k) {
    const int be = tid + k * EWG;
    R[k] = be < NB ? p.rpart[(int64_t)b * NB + be] : 0.f;
  }
  const int any = __syncthreads_or(R[0] > 0.f || R[1] > 0.f);
  int beta = block_stage(NB, p.seed, b, ks, ST_BONUS_BLOCK, sm.ru[0], [&](int, int k) -> float {
    return any ? R[k] : block_w(M[k], S[k], mt, s);
  });
  if (beta < 0) beta = 0;
  const int x0 = beta * BLK + TPT * tid;
  float zt[TPT], zd[TPT];
  load_run<DT, AL>(rt, V, x0, zt);
  load_run<DT, AL>(rd, V, x0, zd);
  const float Mb = sm.M[beta];
  int x = -1;
  if (any) {
    // r = p - sigma > 0 iff d = ln sigma - ln p < 0, and then r = p (-expm1(d))
    const uint32_t smask = F > 0 ? set_mask(p.dtopf + row * p.ld_dtopf, F, x0) : 0u;
    const double invT = ss.invT, D0 = ss.D0, lnC = ss.lnC;
    x = token_race(x0, V, p.seed, b, ks, ST_BONUS_TOKEN, sm.ru[1], [&](int e) -> float {
      if (!(zt[e] > -INFINITY)) return INFINITY;
      const float tp = (Mb - zt[e]) * s;
      if (!(zd[e] > -INFINITY)) return tp;
      const double dd = ((double)zd[e] - (double)zt[e]) * invT + D0 + (((smask >> e) & 1u) ? lnC : 0.0);
      if (!(dd < 0.0)) return INFINITY;
      return tp - __builtin_amdgcn_logf(-expm1f((float)dd));
    });
  }
  if (x < 0) {
    // no residual mass, or the chosen block had mass only through rounding: p there
    x = token_race(x0, V, p.seed, b, ks, ST_BONUS_TOKEN, sm.ru[2], [&](int e) -> float {
      return zt[e] > -INFINITY ? (Mb - zt[e]) * s : INFINITY;
    });
  }
  if (tid == 0) p.bonus[b] = (x >= 0 && x < V) ? x : 0;
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------
// (f32 and unaligned rows need more registers per element: fewer waves)
template <int DT, bool AL, int MODE>
__global__ __launch_bounds__(WG, (DT == SSD_F32 || !AL) ? 4 : 6) void k_stream(Params p) {
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
  RawBlock<DT, AL> r0, r1;
  const bool full = (chunk + 1) * CH * BLK <= V;
  if (full) {
    // every block of this chunk is full: all loads in flight together
    load_raw<DT, AL, true>(rp, V, b0, lane, r0);
    load_raw<DT, AL, true>(rp, V, b1, lane, r1);
  } else {
    // the chunk holding the ragged end of the row
    load_raw<DT, AL, false>(rp, V, min(b0, NB - 1), lane, r0);
    load_raw<DT, AL, false>(rp, V, min(b1, NB - 1), lane, r1);
  }
  float v[32];
  decode_raw<DT, AL>(r0, v);
  const float4 P0 = block_partial<DT, MODE>(v, s, min(b0, NB - 1), lane);
  decode_raw<DT, AL>(r1, v);
  const float4 P1 = block_partial<DT, MODE>(v, s, min(b1, NB - 1), lane);
  if (lane == 0 && b0 < NB) p.part[row * NB + b0] = P0;
  if (lane == 0 && b1 < NB) p.part[row * NB + b1] = P1;
  if constexpr (MODE == M_VERIFY) {
    // the workgroup whose chunk holds x_j hands its target logit to the epilogue
    if (xj >= 0 && xj < V && xj / (CH * BLK) == chunk && threadIdx.x == 0)
      p.zcap[(row / K1) * p.K + (row % K1)] = load_elem<DT>(rp, xj);
  }
}

// One workgroup per row (per sequence for verification) over the partials.
template <int DT, bool AL, int MODE>
__global__ __launch_bounds__(EWG) void k_epi(Params p) {
  __shared__ ESm sm;
  const int g = blockIdx.x;
  if constexpr (MODE == M_VERIFY) epi_verify<DT, AL>(p, g, sm);
  if constexpr (MODE == M_SOFTMAX) epi_softmax<DT, AL>(p, g, sm);
  if constexpr (MODE == M_TOPF) epi_topf<DT, AL>(p, g, sm);
  if constexpr (MODE == M_SAMPLE) epi_sample<DT, AL>(p, g, sm);
}

// Residual pass for sequences rejected at k* < K: block sums of
// max(0, p - sigma) over target row k* and draft row k*, in the target's
// units scaled by exp(L_t) 2^(eps_t) (a constant per sequence).  One block
// per wave; no LDS and no barrier.
template <int DT, bool AL>
__global__ __launch_bounds__(WG, (DT == SSD_F32 || !AL) ? 4 : 5) void k_residual(Params p) {
  const int item = blockIdx.x;
  const int b = item / p.nchunk;
  const int chunk = item - b * p.nchunk;
  const SeqState ss = p.state[b];
  if (!ss.need) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K1 = p.K + 1, V = (int)p.V;
  const int64_t row = (int64_t)b * K1 + ss.kstar;
  const int64_t rs = p.ld * Dt<DT>::SZ;
  const unsigned char* rt = p.x + row * rs;
  const unsigned char* rd = p.xd + row * rs;
  const int be = chunk * CH_R + wave;
  if (be >= p.NB) return;
  float vt[32], vd[32];
  if ((be + 1) * BLK <= V) {
    load_block_full<DT, AL>(rt, be, lane, vt);
    load_block_full<DT, AL>(rd, be, lane, vd);
  } else {
    load_block<DT, AL>(rt, V, be, lane, vt);
    load_block<DT, AL>(rd, V, be, lane, vd);
  }
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
    const int x = p.dtopf[row * p.ld_dtopf + f];
    if (x >= 0 && x < V && x / BLK == be) {
      const float zt = load_elem<DT>(rt, x), zd = load_elem<DT>(rd, x);
      const float e1 = __builtin_amdgcn_exp2f(fmaf(zt, s, ot));
      const float e2 = __builtin_amdgcn_exp2f(fmaf(zd, s, od));
      R += fmaxf(fmaf(nk * p.C, e2, e1), 0.f) - fmaxf(fmaf(nk, e2, e1), 0.f);
    }
  }
  if (lane == 0) p.rpart[(int64_t)b * p.NB + be] = fmaxf(R, 0.f);
}

template <int DT, bool AL>
__global__ __launch_bounds__(EWG) void k_residual_epi(Params p) {
  __shared__ ESm sm;
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
