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

// Phase stamps of the latency-bound kernels, compiled in only for the
// instrumented build (-DSSD_PHASES, a measurement aid): the first lane of
// wave 0 records the 100 MHz real-time counter at fixed points of each item
// (kind 0: sampling epilogue, per row; kind 1: verification after the
// streaming pass, per sequence).  The stamps are kept in registers and
// stored at the end of the item, so that no stamp's store is outstanding
// while the item waits on a load (one wait counter covers loads and stores).
constexpr int PH_N = 8;
constexpr int PH_ITEMS = 8192;
#ifdef SSD_PHASES
__device__ uint64_t g_phase[2][PH_ITEMS * PH_N];
#define SSD_PH_DECL uint64_t ph_[PH_N] = {}
#define SSD_PH(k) (ph_[k] = __builtin_amdgcn_s_memrealtime())
#define SSD_PH_SET(k, v) (ph_[k] = (uint64_t)(v))
#define SSD_PH_FLUSH(kind, item)                                                              \
  do {                                                                                        \
    if (threadIdx.x == 0 && (int64_t)(item) < PH_ITEMS)                                       \
      for (int k_ = 0; k_ < PH_N; ++k_) g_phase[kind][(int64_t)(item) * PH_N + k_] = ph_[k_];  \
  } while (0)
#else
#define SSD_PH_DECL \
  do {              \
  } while (0)
#define SSD_PH(k) \
  do {            \
  } while (0)
#define SSD_PH_SET(k, v) \
  do {                   \
  } while (0)
#define SSD_PH_FLUSH(kind, item) \
  do {                           \
  } while (0)
#endif

enum Mode { M_SOFTMAX = 0, M_TOPF = 1, M_SAMPLE = 2, M_VERIFY = 3 };

constexpr int CH = 8;             // blocks per workgroup in the streaming pass (2 per wave)
constexpr int CH_R = 2 * EWG / 64;  // blocks per pass of a workgroup over a residual (2 per wave)
constexpr int TPT = BLK / EWG;    // tokens per epilogue thread in a token stage
constexpr int NBT = MAX_NB / EWG; // blocks per epilogue thread
constexpr int NBL = MAX_NB / 64;  // blocks per lane when a wave holds a whole row
static_assert(TPT == 8 && NBT == 2, "epilogue layout assumes 256 threads over 2048-token blocks");
constexpr int KTH_ROUNDS = 8;     // top-F threshold by maximum rounds up to this F, by radix search above
constexpr int TF_CAP = EWG;       // (K+1)*F draft top-F entries prefetched into LDS when they fit

// Constants of the bonus draw from the residual of one sequence's row k*.
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
  int jlo, jn;              // jn > 0: the streaming pass covers positions jlo .. jlo + jn - 1 of every sequence
  int early;                // verification: rows past the first rejection may not have been streamed
  int keep;                 // verification: positions < keep are streamed with ordinary (cached) loads
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
  int32_t* gate;            // early exit: [0] the number of sequences the gate keeps, [1 + i] the i-th of them [1 + B]
  int gate_reset;           // verification stream: the first workgroup sets gate[0] to 0
  // speculation cache (optional): depth offsets, keys, payload, lookup outputs
  int koff[MAX_K1 + 1];
  int Bgt;
  int fill;                 // verification: a miss gets the random fallback tokens (else -1)
  int kdep[MAX_K1];         // sampling: depths whose key list is longer than F_sel, each ranked by
  int nkd;                  // B extra workgroups of the epilogue (after the B (K+1) row workgroups)
  int lookup;               // verification looks (k*, bonus) up
  int32_t* ckeys;           // [B, Bgt]; sampling writes, verification reads
  const int32_t* cpay;      // [B, Bgt, K]
  int32_t* chit;
  int32_t* cslot;
  int32_t* ctok;
};

// LDS of an epilogue workgroup.
// The top-F selection's plan, set by wave 0 for the workgroup: whether
// candidate blocks are re-read, the one-element candidates listed, the
// candidate and re-read block counts, the threshold.
struct TopfQ {
  int reread, n1, ncb, nrb;
  float tau;
};
struct ESm {
  float rf[2][ENW];         // reduction slots, one per call site
  double rd[2][ENW];
  uint64_t ru[6][ENW];
  int ri[2][ENW];
  float M[MAX_NB];          // block maxima (verification: row K; residual: target row k*)
  float S[MAX_NB];          // block sums (verification: row K)
  int cblk[MAX_NB];         // candidate blocks for top-F
  int rblk[MAX_NB];         // candidate blocks re-read for top-F
  uint64_t cand[CAND_CAP];  // top-F candidates as (value desc, index asc) keys
  uint64_t tkey[MAX_F];     // top-F result through LDS, sorted
  uint64_t wk[ENW][64];     // each wave's own top-F exchange row
  TopfQ tq;                 // top-F plan (wave 0)
  int tf[TF_CAP];           // verification: the draft top-F lists of a sequence's rows
  int nre;                  // candidates appended by block re-reads
  int ks;
  int bonus;
  SeqState ss;
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
// epilogue building blocks.  An epilogue workgroup has ENW waves.  Each wave
// holds its own copy of a row's partials in registers (block be = lane + 64*i
// in slot i < PLN), so the row maximum and sum, the top-F threshold and the
// block draw are computed by every wave without a barrier; the waves split
// only the 2048-token stage.
// ---------------------------------------------------------------------------
template <int PLN>
struct WRow {
  float M[PLN], S[PLN], M2[PLN];
  int I[PLN];
};

template <int PLN>
__device__ __forceinline__ void load_wrow(const float4* pr, int NB, WRow<PLN>& r) {
  const int lane = threadIdx.x & 63;
  // unconditional loads from clamped addresses, so that every slot's load is
  // in flight at once (a load under a branch gets a wait of its own)
  float4 v[PLN];
#pragma unroll
  for (int i = 0; i < PLN; ++i) v[i] = pr[min(lane + 64 * i, NB - 1)];
#pragma unroll
  for (int i = 0; i < PLN; ++i) {
    const bool in = lane + 64 * i < NB;
    r.M[i] = in ? v[i].x : -INFINITY;
    r.S[i] = in ? v[i].y : 0.f;
    r.I[i] = in ? __float_as_int(v[i].z) : -1;
    r.M2[i] = in ? v[i].w : -INFINITY;
  }
}

// Entry be (uniform) of a slot array, read from the lane that holds it.
template <int PLN, class Tv>
__device__ __forceinline__ Tv slot_at(const Tv (&x)[PLN], int be) {
  Tv r = x[0];
#pragma unroll
  for (int i = 0; i < PLN; ++i) {
    const Tv y = __builtin_bit_cast(Tv, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x[i]), be & 63));
    r = (i == (be >> 6)) ? y : r;
  }
  return r;
}

// Low bits of the order-preserving key that only repeat the sign: a bf16
// value widened to binary32 has 16 zero low bits, an fp16 value 13.
template <int DT> struct LowBit { static constexpr int B = 0; };
template <> struct LowBit<SSD_BF16> { static constexpr int B = 16; };
template <> struct LowBit<SSD_F16> { static constexpr int B = 13; };

// The Fs-th largest of the wave's keys (absent slots hold 0): the largest c
// with at least Fs keys >= c.  The keys lie in [kmin, kmax], so the answer
// shares their common high bits; the bits below are found two at a time by
// counting keys at or above three trial values with ballots.
template <int PLN>
__device__ __forceinline__ uint32_t kth_key(const uint32_t (&key)[PLN], int Fs, uint32_t kmax, uint32_t kmin,
                                            int lowbit) {
  const uint32_t diff = kmax ^ kmin;
  if (diff == 0) return kmax;
  const int hb = 31 - __builtin_clz(diff);
  uint32_t tk = kmax & ~((2u << hb) - 1u);
  int bit = hb;
  for (; bit - 1 >= lowbit; bit -= 2) {
    const uint32_t c1 = tk | (1u << (bit - 1)), c2 = tk | (2u << (bit - 1)), c3 = tk | (3u << (bit - 1));
    int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
    for (int i = 0; i < PLN; ++i) {
      n1 += __popcll(__ballot(key[i] >= c1));
      n2 += __popcll(__ballot(key[i] >= c2));
      n3 += __popcll(__ballot(key[i] >= c3));
    }
    tk = n3 >= Fs ? c3 : n2 >= Fs ? c2 : n1 >= Fs ? c1 : tk;
  }
  if (bit >= lowbit) {
    const uint32_t c = tk | (1u << bit);
    int n = 0;
#pragma unroll
    for (int i = 0; i < PLN; ++i) n += __popcll(__ballot(key[i] >= c));
    if (n >= Fs) tk = c;
  }
  if (lowbit > 0 && !(tk & 0x80000000u)) tk |= (1u << lowbit) - 1u;  // negative values: low bits all ones
  return tk;
}

// The same for small Fs: rounds of a wave maximum, each removing every copy
// of the largest remaining key and counting them, until Fs keys are counted
// (at most Fs rounds, each a short DPP reduction instead of a chain of
// ballot counts per bit pair).
template <int PLN>
__device__ __forceinline__ uint32_t kth_key_rounds(const uint32_t (&key)[PLN], int Fs) {
  uint32_t k[PLN];
#pragma unroll
  for (int i = 0; i < PLN; ++i) k[i] = key[i];
  uint32_t mx = 0;
  int cum = 0;
  for (int r = 0; r < Fs; ++r) {
    uint32_t lm = k[0];
#pragma unroll
    for (int i = 1; i < PLN; ++i) lm = max(lm, k[i]);
    mx = wave_max_u32(lm);
#pragma unroll
    for (int i = 0; i < PLN; ++i) cum += __popcll(__ballot(k[i] == mx));
    if (cum >= Fs || mx == 0u) break;
#pragma unroll
    for (int i = 0; i < PLN; ++i) k[i] = k[i] == mx ? 0u : k[i];
  }
  return mx;
}

// Exact top-Fs of a row (value desc, index asc) from a wave's copy of its
// partials.  The block maxima and second values are values of 2 NB distinct
// elements, so tau, the Fs-th largest of them, bounds the Fs-th largest
// element from below, and every top element lies in a candidate block
// (maximum >= tau).  A candidate whose second value is below tau holds
// exactly one element >= tau, its maximum, whose index the partial carries.
// When every candidate is of that kind (the common case) the wave ranks the
// candidate maxima itself; otherwise the other candidates are re-read by the
// whole workgroup (each thread one 16-byte chunk of each) and all candidates
// are ranked through LDS.  sm.nre must have been cleared at start.
//
// topf_plan (one wave, or every wave with the same copy): tau and the
// candidates.  In the common case it writes the ranked list to out[0 .. Fs)
// and returns true; otherwise wave 0 lists the candidate blocks, the blocks
// to re-read and the one-element candidates with the plan in sm.tq, and it
// returns false.
template <int DT, bool AL, int PLN>
__device__ __forceinline__ bool topf_plan(int NB, int Fs, const WRow<PLN>& r, float m, ESm& sm, uint64_t* out) {
  const int lane = threadIdx.x & 63;
  const bool w0 = threadIdx.x < 64;
  // the block maxima and second values: 2 NB values of distinct elements
  // (a second value of -inf in a one-element block stands for none)
  uint32_t key[2 * PLN];
  uint32_t kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < PLN; ++i) {
    const bool in = lane + 64 * i < NB;
    key[i] = in ? ord_key(r.M[i]) : 0u;
    key[PLN + i] = in ? ord_key(r.M2[i]) : 0u;
    kmin = in ? min(kmin, key[PLN + i]) : kmin;
  }
  const bool sel = 2 * NB > Fs;
  const uint32_t tk = !sel ? 0u
                    : Fs <= KTH_ROUNDS ? kth_key_rounds<2 * PLN>(key, Fs)
                                       : kth_key<2 * PLN>(key, Fs, ord_key(m), wave_min_u32(kmin), LowBit<DT>::B);
  const float tau = sel ? ord_val(tk) : -INFINITY;
  bool cand[PLN], one[PLN];
  uint64_t more = 0;
#pragma unroll
  for (int i = 0; i < PLN; ++i) {
    cand[i] = lane + 64 * i < NB && key[i] >= tk;
    one[i] = cand[i] && sel && r.M2[i] < tau;
    more |= __ballot(cand[i] && !one[i]);
  }
  if (more == 0) {
    // every candidate holds one element >= tau: rank the candidate maxima
    uint64_t ck[PLN];
    int rk[PLN];
#pragma unroll
    for (int i = 0; i < PLN; ++i) {
      ck[i] = cand[i] ? vi_key(r.M[i], r.I[i]) : 0ull;
      rk[i] = 0;
    }
#pragma unroll
    for (int i = 0; i < PLN; ++i) {
      uint64_t mk = __ballot(cand[i]);
      while (mk) {
        const uint64_t kc = rl_u64(ck[i], (int)__builtin_ctzll(mk));
        mk &= mk - 1ull;
#pragma unroll
        for (int i2 = 0; i2 < PLN; ++i2) rk[i2] += kc > ck[i2];  // candidates ranked above
      }
    }
#pragma unroll
    for (int i = 0; i < PLN; ++i)
      if (cand[i] && rk[i] < Fs) out[rk[i]] = ck[i];
    if (w0 && lane == 0) sm.tq.reread = 0;
    return true;
  } else {
    // the candidate blocks, the blocks to re-read and the one-element
    // candidates, listed for the whole workgroup
    const uint64_t below = (1ull << lane) - 1ull;
    int n1 = 0, ncb = 0, nrb = 0;
#pragma unroll
    for (int i = 0; i < PLN; ++i) {
      const int be = lane + 64 * i;
      const bool re = cand[i] && !one[i];
      const uint64_t cm = __ballot(cand[i]), om = __ballot(one[i]), rm = __ballot(re);
      if (w0 && cand[i]) sm.cblk[ncb + __popcll(cm & below)] = be;
      if (w0 && re) sm.rblk[nrb + __popcll(rm & below)] = be;
      if (w0 && one[i] && n1 + __popcll(om & below) < CAND_CAP)
        sm.cand[n1 + __popcll(om & below)] = vi_key(r.M[i], r.I[i]);
      ncb += __popcll(cm);
      n1 += __popcll(om);
      nrb += __popcll(rm);
    }
    if (w0 && lane == 0) sm.tq = TopfQ{1, n1, ncb, nrb, tau};
    return false;
  }
}

// The whole workgroup, after a barrier that follows topf_plan's false: every
// thread scans its 16-byte chunks of the re-read blocks and all candidates
// are ranked into sm.tkey; ends with a barrier.
template <int DT, bool AL>
__device__ __forceinline__ void topf_reread(const unsigned char* rp, int V, int Fs, ESm& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const TopfQ q = sm.tq;
  // every thread scans its 16-byte chunks of the re-read blocks, RB blocks'
  // loads in flight at a time
  const float tau = q.tau;
  const int n1 = q.n1, ncb = q.ncb, nrb = q.nrb;
  {
    constexpr int VW = Dt<DT>::VW, RB = 8;
    for (int c0 = tid; c0 < BLK / VW; c0 += EWG) {  // chunk c0 of every re-read block
      for (int k0 = 0; k0 < nrb; k0 += RB) {
        float v[RB][VW];
        if constexpr (AL) {
          // all RB loads are issued before any is decoded (left to itself the
          // scheduler interleaves them with the decoding, two loads in flight)
          uint4 w[RB];
#pragma unroll
          for (int u = 0; u < RB; ++u) {
            const int e0 = sm.rblk[min(k0 + u, nrb - 1)] * BLK + c0 * VW;
            w[u] = *reinterpret_cast<const uint4*>(rp + (size_t)(e0 < V ? e0 : 0) * Dt<DT>::SZ);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < RB; ++u) {
            const int e0 = sm.rblk[min(k0 + u, nrb - 1)] * BLK + c0 * VW;
            decode16<DT>(w[u], v[u]);
#pragma unroll
            for (int e = 0; e < VW; ++e) v[u][e] = e0 < V ? v[u][e] : -INFINITY;
          }
        } else {
#pragma unroll
          for (int u = 0; u < RB; ++u) {
            const int e0 = sm.rblk[min(k0 + u, nrb - 1)] * BLK + c0 * VW;
            load_chunk<DT, AL>(rp, V, e0, v[u]);
          }
        }
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          if (k0 + u >= nrb) break;
          const int e0 = sm.rblk[k0 + u] * BLK + c0 * VW;
#pragma unroll
          for (int e = 0; e < VW; ++e) {
            if (v[u][e] >= tau && e0 + e < V) {
              const int pos = n1 + atomicAdd(&sm.nre, 1);
              if (pos < CAND_CAP) sm.cand[pos] = vi_key(v[u][e], e0 + e);
            }
          }
        }
      }
    }
  }
  lds_sync();
  const int n = n1 + sm.nre;
  if (n <= CAND_CAP) {
    for (int c = tid; c < n; c += EWG) {
      const uint64_t ki = sm.cand[c];
      int rk = 0, c2 = 0;
      for (; c2 + 4 <= n; c2 += 4)
        rk += (sm.cand[c2] > ki) + (sm.cand[c2 + 1] > ki) + (sm.cand[c2 + 2] > ki) + (sm.cand[c2 + 3] > ki);
      for (; c2 < n; ++c2) rk += sm.cand[c2] > ki;
      if (rk < Fs) sm.tkey[rk] = ki;
    }
  } else {
    // More than CAND_CAP elements at or above tau (a short row with a long
    // list, or many ties): the Fs-th largest key by a radix select over the
    // candidate blocks' elements, eight bits a round from the top (a 256-bin
    // histogram in LDS of the keys that share the bits fixed so far), until
    // the keys sharing the prefix are exactly the ones still needed; then
    // those keys and every larger one (Fs in all) are collected and ranked.
    constexpr int VW = Dt<DT>::VW;
    static_assert(EWG == 256, "one histogram bin per thread");
    int* hist = reinterpret_cast<int*>(sm.cand);  // (the candidate list is not read here)
    auto scan = [&](auto&& fn) {
      for (int c = 0; c < ncb; ++c) {
        const int be = sm.cblk[c];
        for (int c0 = tid; c0 < BLK / VW; c0 += EWG) {
          const int e0 = be * BLK + c0 * VW;
          float v[VW];
          load_chunk<DT, AL>(rp, V, e0, v);
#pragma unroll
          for (int e = 0; e < VW; ++e)
            if (v[e] >= tau && e0 + e < V) fn(vi_key(v[e], e0 + e));
        }
      }
    };
    uint64_t prefix = 0, pmask = 0;
    int need = Fs;
    for (int sh = 56; sh >= 0; sh -= 8) {
      hist[tid] = 0;
      lds_sync();
      scan([&](uint64_t k) {
        if ((k & pmask) == prefix) atomicAdd(&hist[(int)(k >> sh) & 255], 1);
      });
      lds_sync();
      if (wave == 0) {
        // lane l holds bins 4l .. 4l+3; the need-th largest key of the
        // prefix lies in the highest lane whose bins and those above reach
        // need, in the highest of its bins that reaches it
        int h[4], hs = 0;
#pragma unroll
        for (int b2 = 0; b2 < 4; ++b2) {
          h[b2] = hist[4 * lane + b2];
          hs += h[b2];
        }
        int suf = hs;  // bins of lanes >= l
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int t = __shfl_down(suf, off);
          suf += lane + off < 64 ? t : 0;
        }
        const uint64_t reach = __ballot(suf >= need);
        const int ls = 63 - (int)__builtin_clzll(reach);  // reach != 0: the prefix's keys number >= need
        if (lane == ls) {
          int cum = suf - hs, d = 4 * lane, hd = h[0];
#pragma unroll
          for (int b2 = 3; b2 >= 0; --b2) {
            if (cum + h[b2] >= need) {
              d = 4 * lane + b2;
              hd = h[b2];
              break;
            }
            cum += h[b2];
          }
          sm.ri[0][0] = d;
          sm.ri[0][1] = cum;
          sm.ri[0][2] = hd;
        }
      }
      lds_sync();
      const int d = sm.ri[0][0], above = sm.ri[0][1], hd = sm.ri[0][2];
      need -= above;
      prefix |= (uint64_t)d << sh;
      pmask |= 255ull << sh;
      if (hd == need) break;  // uniform: every thread read the same values
    }
    // the Fs keys: those above the prefix and those sharing it
    if (tid == 0) sm.ri[1][0] = 0;
    lds_sync();
    scan([&](uint64_t k) {
      if ((k & pmask) >= prefix) {
        const int pos = atomicAdd(&sm.ri[1][0], 1);
        if (pos < Fs) sm.cand[pos] = k;
      }
    });
    lds_sync();
    for (int c = tid; c < Fs; c += EWG) {
      const uint64_t ki = sm.cand[c];
      int rk = 0;
      for (int c2 = 0; c2 < Fs; ++c2) rk += sm.cand[c2] > ki;
      sm.tkey[rk] = ki;
    }
  }
  lds_sync();
}

// Every wave with its own copy of the partials: in the common case each
// wave ranks the candidates itself and returns without a barrier (latency
// first: the sampling epilogue's draw goes on in every wave).
template <int DT, bool AL, int PLN>
__device__ __forceinline__ uint64_t wave_topf(const unsigned char* rp, int V, int NB, int Fs, const WRow<PLN>& r,
                                              float m, ESm& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t* wk = sm.wk[wave];
  if (topf_plan<DT, AL, PLN>(NB, Fs, r, m, sm, wk)) {
    // lanes of one wave exchange through their own LDS rows: LDS executes a
    // wave's accesses in order; the fences keep the compiler from reordering
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return lane < Fs ? wk[lane] : 0ull;
  }
  lds_sync();
  topf_reread<DT, AL>(rp, V, Fs, sm);
  return lane < Fs ? sm.tkey[lane] : 0ull;
}

// Wave 0 alone plans the selection from its copy of the partials while the
// other waves wait (throughput first: workgroups whose only output is the
// list).
template <int DT, bool AL, int PLN>
__device__ __forceinline__ uint64_t wg_topf(const unsigned char* rp, int V, int NB, int Fs, const WRow<PLN>& r,
                                            float m, ESm& sm) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) topf_plan<DT, AL, PLN>(NB, Fs, r, m, sm, sm.tkey);
  lds_sync();
  if (sm.tq.reread) topf_reread<DT, AL>(rp, V, Fs, sm);
  return lane < Fs ? sm.tkey[lane] : 0ull;
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

// Block stage over blocks owned by threads (thread t: blocks t + k*EWG):
// argmin of -log2(u_be) / W_be (the common factor ln 2 dropped); wfn(be)
// gives W_be >= 0.  Returns the chosen block, -1 if no block has mass.
template <class WF>
__device__ __forceinline__ int block_stage(int NB, uint64_t seed, int b, int j, uint32_t st, uint64_t* slot,
                                           WF wfn) {
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
// The TPT tokens x0 .. x0 + TPT - 1 of a token stage (past V: -inf), in two
// steps so that independent work can be placed while the loads are in
// flight: run_issue starts the loads, run_finish decodes.  On the aligned
// path the row holds 16-byte chunks (V and x0 are multiples of the chunk,
// so a chunk lies wholly inside the row or wholly past it), loaded
// unconditionally from clamped addresses (a load under a branch gets a wait
// of its own).
template <int DT, bool AL>
struct Run {
  static constexpr int VW = Dt<DT>::VW, NC = TPT / VW;
  uint4 w[AL ? NC : 1];
  float z[AL ? 1 : TPT];
};
template <int DT, bool AL>
__device__ __forceinline__ void run_issue(const unsigned char* rp, int V, int x0, Run<DT, AL>& r) {
  if constexpr (AL) {
#pragma unroll
    for (int c = 0; c < Run<DT, AL>::NC; ++c) {
      const int e0 = x0 + c * Run<DT, AL>::VW;
      r.w[c] = *reinterpret_cast<const uint4*>(rp + (size_t)(e0 < V ? e0 : 0) * Dt<DT>::SZ);
    }
  } else {
#pragma unroll
    for (int e = 0; e < TPT; ++e) {
      const bool in = x0 + e < V;
      const float x = load_elem<DT>(rp, in ? x0 + e : 0);
      r.z[e] = in ? x : -INFINITY;
    }
  }
}
template <int DT, bool AL>
__device__ __forceinline__ void run_finish(int V, int x0, const Run<DT, AL>& r, float (&z)[TPT]) {
  if constexpr (AL) {
    constexpr int VW = Run<DT, AL>::VW;
#pragma unroll
    for (int c = 0; c < Run<DT, AL>::NC; ++c) {
      const int e0 = x0 + c * VW;
      decode16<DT>(r.w[c], &z[c * VW]);
#pragma unroll
      for (int e = 0; e < VW; ++e) z[c * VW + e] = e0 < V ? z[c * VW + e] : -INFINITY;
    }
  } else {
#pragma unroll
    for (int e = 0; e < TPT; ++e) z[e] = r.z[e];
  }
}

// The Philox words of a token stage's TPT tokens (stream st at (b, j)).
struct RaceWords {
  uint32_t w[TPT];
};
__device__ __forceinline__ RaceWords race_words(int x0, uint64_t seed, int b, int j, uint32_t st) {
  const uint4 wa = draws4(seed, (uint32_t)(x0 >> 2), (uint32_t)b, (uint32_t)j, st);
  const uint4 wb = draws4(seed, (uint32_t)(x0 >> 2) + 1u, (uint32_t)b, (uint32_t)j, st);
  return RaceWords{{wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w}};
}

// Token stage of the two-level draw over a block: thread t holds tokens
// x0 .. x0 + TPT - 1 (x0 = beta*BLK + TPT*t) with their Philox words rw; tfn(e)
// gives the log2 of the inverse weight of token x0 + e up to a constant
// common to the block (+inf excludes it).  Returns the winner (-1 if none).
template <class TF>
__device__ __forceinline__ int token_race(int x0, int V, const RaceWords& rw, uint64_t* slot, TF tfn) {
  const uint32_t* w = rw.w;
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

// Bit e set when token x0 + e is one of the first F entries of a top list
// held as lane f = entry f (idx), or in memory (ptr).
__device__ __forceinline__ uint32_t set_mask_lanes(int idx, int F, int x0) {
  uint32_t msk = 0;
  for (int f = 0; f < F; ++f) {
    const uint32_t d = (uint32_t)(__builtin_amdgcn_readlane(idx, f) - x0);
    if (d < (uint32_t)TPT) msk |= 1u << d;
  }
  return msk;
}
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
template <int DT, bool AL, int PLN>
__device__ __forceinline__ void epi_softmax_p(const Params& p, int64_t row) {
  if (threadIdx.x >= 64) return;  // one wave per row
  const int lane = threadIdx.x;
  const float T = p.temp[row];
  const bool greedy = !(T > 0.f);
  const float s = greedy ? 0.f : (float)(LOG2E / (double)T);
  const int NB = p.NB;
  WRow<PLN> r;
  load_wrow<PLN>(p.part + row * NB, NB, r);
  float lm = r.M[0];
#pragma unroll
  for (int i = 1; i < PLN; ++i) lm = fmaxf(lm, r.M[i]);
  const float m = wave_max(lm);
  double w = 0.0;
  int am = -1;
#pragma unroll
  for (int i = PLN - 1; i >= 0; --i) {
    if (!greedy) w += (double)block_w(r.M[i], r.S[i], m, s);
    const uint64_t mk = __ballot(lane + 64 * i < NB && r.M[i] == m);
    if (mk) am = __builtin_amdgcn_readlane(r.I[i], (int)__builtin_ctzll(mk));  // first block holding m
  }
  const double tot = greedy ? 1.0 : wave_sum_d(w);
  if (lane == 0) {
    ssd_row_stats st;
    st.lse = greedy ? 0.0 : ln_fast(tot);
    st.max = m;
    st.argmax = am < 0 ? 0 : am;  // (a NaN row matches no block)
    p.stats[row] = st;
  }
}

template <int DT, bool AL, int PLN>
__device__ __forceinline__ void epi_topf_p(const Params& p, int64_t row, ESm& sm) {
  if (threadIdx.x == 0) sm.nre = 0;
  const int NB = p.NB;
  WRow<PLN> r;
  float m = 0.f;
  if (threadIdx.x < 64) {  // wave 0's copy of the partials serves the selection
    load_wrow<PLN>(p.part + row * NB, NB, r);
    float lm = r.M[0];
#pragma unroll
    for (int i = 1; i < PLN; ++i) lm = fmaxf(lm, r.M[i]);
    m = wave_max(lm);
  }
  const uint64_t tk = wg_topf<DT, AL, PLN>(p.x + row * p.ld * Dt<DT>::SZ, (int)p.V, NB, p.F, r, m, sm);
  const int lane = threadIdx.x;
  if (lane < p.F) {  // wave 0 only: lane < F <= 64
    p.out_idx[row * p.F + lane] = (int)key_idx(tk);
    if (p.out_val) p.out_val[row * p.F + lane] = key_val(tk);
  }
}

template <int DT, bool AL, int PLN>
__device__ __forceinline__ void epi_sample_p(const Params& p, int64_t row, ESm& sm) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int K1 = p.K + 1;
  const int b = (int)(row / K1), j = (int)(row % K1);
  const float T = p.temp[b];
  const bool greedy = !(T > 0.f);
  const float s = greedy ? 0.f : (float)(LOG2E / (double)T);
  const int NB = p.NB, V = (int)p.V, F = p.F;
  const float C = p.C;
  const unsigned char* rp = p.x + row * p.ld * Dt<DT>::SZ;
  SSD_PH_DECL;
  SSD_PH(0);
  if (tid == 0) sm.nre = 0;
  const bool draw = !greedy && j < p.K;
  WRow<PLN> r;
  load_wrow<PLN>(p.part + row * NB, NB, r);
  // -log2(u) of every block for the block stage: independent of the logits,
  // computed while the partials load
  float E[PLN];
#pragma unroll
  for (int i = 0; i < PLN; ++i)
    E[i] = draw ? neg_log2_u(draw1(p.seed, (uint32_t)(lane + 64 * i), (uint32_t)b, (uint32_t)j, ST_DRAFT_BLOCK))
                : 0.f;
  float lm = r.M[0];
#pragma unroll
  for (int i = 1; i < PLN; ++i) lm = fmaxf(lm, r.M[i]);
  const float m = wave_max(lm);
  SSD_PH(1);  // partials loaded, row maximum
  float w[PLN];
  double ws = 0.0;
#pragma unroll
  for (int i = 0; i < PLN; ++i) {
    w[i] = greedy ? 0.f : block_w(r.M[i], r.S[i], m, s);
    ws += (double)w[i];
  }
  const double tot0 = greedy ? 1.0 : wave_sum_d(ws);
  SSD_PH(2);  // block weights and their sum
  // entries ranked: F for sigma and F_out listed; this depth's cache keys
  // when they fit in that list (longer key lists have workgroups of their own)
  const int Fj = p.ckeys ? p.koff[j + 1] - p.koff[j] : 0;
  const uint64_t tkey = wave_topf<DT, AL, PLN>(rp, V, NB, p.F_sel, r, m, sm);
  SSD_PH(3);  // top-F list
  const float tv = key_val(tkey);
  const int ti = (int)key_idx(tkey);
  // sigma_{F,C}: lane f < F holds 2^((z_f - m) s) of the f-th member of S
  const float es = (!greedy && lane < F) ? __builtin_amdgcn_exp2f((tv - m) * s) : 0.f;
  const double zs = wave_sum_d((double)es);
  const double lse = greedy ? 0.0 : ln_fast((tot0 - zs) + (double)C * zs);
  // the row's outputs are stored at the end of each path: a wait for a later
  // load (the chosen block's) would wait for them too (one counter covers
  // loads and stores)
  auto store_row = [&]() {
    if (tid < 64) {
      if (lane < p.F_out) {
        if (p.out_idx) p.out_idx[row * p.F_out + lane] = ti;
        if (p.out_val) p.out_val[row * p.F_out + lane] = tv;
      }
      if (Fj <= p.F_sel && lane < Fj) p.ckeys[(int64_t)b * p.Bgt + p.koff[j] + lane] = ti;
      if (lane == 0) {
        ssd_row_stats st;
        st.lse = lse;
        st.max = m;
        st.argmax = ti;
        p.stats[row] = st;
      }
    }
  };
  SSD_PH(4);  // sigma normaliser
  if (j == p.K) {  // row K only predicts the bonus after K acceptances
    store_row();
    SSD_PH_FLUSH(0, row);
    return;
  }
  if (greedy) {
    if (tid == 0) {
      p.tokens[b * p.K + j] = ti;
      p.q[b * p.K + j] = 1.0f;
    }
    store_row();
    SSD_PH_FLUSH(0, row);
    return;
  }
  // block stage (every wave): blocks holding members of S lose (1 - C) of
  // those members' weight
  float corr[PLN];
#pragma unroll
  for (int i = 0; i < PLN; ++i) corr[i] = 0.f;
  for (int f = 0; f < F; ++f) {
    const int bf = __builtin_amdgcn_readlane(ti, f) / BLK;
    const float ef = rl_f(es, f);
#pragma unroll
    for (int i = 0; i < PLN; ++i) corr[i] += (bf == lane + 64 * i) ? ef : 0.f;
  }
  uint64_t bk = NO_KEY;
#pragma unroll
  for (int i = 0; i < PLN; ++i) {
    const float W = corr[i] > 0.f ? fmaxf(w[i] - corr[i], 0.f) + C * corr[i] : w[i];
    if (lane + 64 * i < NB && W > 0.f) bk = umin64(bk, race_key(E[i] * __builtin_amdgcn_rcpf(W), lane + 64 * i));
  }
  bk = wave_min_u64(bk);
  const int beta = bk == NO_KEY ? 0 : (int)(uint32_t)bk;  // no block of mass only for invalid rows
  SSD_PH(5);  // block drawn
  // token stage over block beta
  const int x0 = beta * BLK + TPT * tid;
  Run<DT, AL> run;
  run_issue<DT, AL>(rp, V, x0, run);
  const RaceWords rw = race_words(x0, p.seed, b, j, ST_DRAFT_TOKEN);  // while the block loads
  const uint32_t smask = set_mask_lanes(ti, F, x0);
  __builtin_amdgcn_sched_barrier(0);
  float z[TPT];
  run_finish<DT, AL>(V, x0, run, z);
  const float nc2 = -__builtin_amdgcn_logf(C);  // -log2 C >= 0
  const float Mb = slot_at<PLN>(r.M, beta);
  const int x = token_race(x0, V, rw, sm.ru[1], [&](int e) -> float {
    if (!(z[e] > -INFINITY)) return INFINITY;
    return (Mb - z[e]) * s + (((smask >> e) & 1u) ? nc2 : 0.f);
  });
  SSD_PH(6);  // chosen block re-read and token race
  const uint32_t d = (uint32_t)(x - x0);
  if (x >= 0 && d < (uint32_t)TPT) {
    // the owner of the winning token writes it with sigma_j(x)
    float zx = z[0];
#pragma unroll
    for (int e = 1; e < TPT; ++e) zx = (d == (uint32_t)e) ? z[e] : zx;
    const bool inS = (smask >> d) & 1u;
    const double lq = ((double)zx - (double)m) * (1.0 / (double)T) + (inS ? ln_fast((double)C) : 0.0) - lse;
    p.tokens[b * p.K + j] = x;
    p.q[b * p.K + j] = __builtin_amdgcn_exp2f((float)(lq * LOG2E));
  } else if (x < 0 && tid == 0) {
    p.tokens[b * p.K + j] = 0;
    p.q[b * p.K + j] = 0.f;
  }
  store_row();
  SSD_PH_FLUSH(0, row);
}

// Cache keys of depth kdep[item / B] for sequence item % B: the first F_j
// entries of that draft row's top list (a workgroup of its own, in parallel
// with the row's sampling).
template <int DT, bool AL, int PLN>
__device__ __forceinline__ void epi_keys_p(const Params& p, int item, ESm& sm) {
  const int b = item % p.B, j = p.kdep[item / p.B];
  const int64_t row = (int64_t)b * (p.K + 1) + j;
  const int Fj = p.koff[j + 1] - p.koff[j];
  if (threadIdx.x == 0) sm.nre = 0;
  const int NB = p.NB;
  WRow<PLN> r;
  float m = 0.f;
  if (threadIdx.x < 64) {  // wave 0's copy of the partials serves the selection
    load_wrow<PLN>(p.part + row * NB, NB, r);
    float lm = r.M[0];
#pragma unroll
    for (int i = 1; i < PLN; ++i) lm = fmaxf(lm, r.M[i]);
    m = wave_max(lm);
  }
  const uint64_t tk = wg_topf<DT, AL, PLN>(p.x + row * p.ld * Dt<DT>::SZ, (int)p.V, NB, Fj, r, m, sm);
  const int lane = threadIdx.x;
  if (lane < Fj) p.ckeys[(int64_t)b * p.Bgt + p.koff[j] + lane] = (int)key_idx(tk);  // wave 0: Fj <= 64
}

// Residual block sum sum_x max(0, p_x - c sigma_x) over block be of one row,
// in the target's units (one wave; every lane gets the sum).  ut and ud hold
// the block of the target and draft rows; e1 = 2^(z_t s + ot) and e2 =
// 2^(z_d s + od); nk = -c times the draft term in the target's units and nkc
// = nk C for the members of the draft's top-F set (tfl: F entries, in LDS or
// global memory), whose terms are corrected one by one.  The member's logits
// are element kk of lane gi & 63 in the wave's registers.
template <int DT, bool AL>
__device__ __forceinline__ float block_residual(const RawBlock<DT, AL>& ut, const RawBlock<DT, AL>& ud, int be, int V,
                                                float s, float ot, float od, float nk, float nkc, int F,
                                                const int32_t* tfl) {
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int k = 0; k < 32; k += 2) {
    const float e1 = __builtin_amdgcn_exp2f(fmaf(raw_elem<DT, AL>(ut, k), s, ot));
    const float e2 = __builtin_amdgcn_exp2f(fmaf(raw_elem<DT, AL>(ud, k), s, od));
    const float f1 = __builtin_amdgcn_exp2f(fmaf(raw_elem<DT, AL>(ut, k + 1), s, ot));
    const float f2 = __builtin_amdgcn_exp2f(fmaf(raw_elem<DT, AL>(ud, k + 1), s, od));
    a0 += fmaxf(fmaf(nk, e2, e1), 0.f);
    a1 += fmaxf(fmaf(nk, f2, f1), 0.f);
  }
  float R = wave_sum(a0 + a1);
  for (int f = 0; f < F; ++f) {
    const int x = __builtin_amdgcn_readfirstlane(tfl[f]);
    if (x >= 0 && x < V && x / BLK == be) {
      constexpr int VW = Dt<DT>::VW;
      const int off = x - be * BLK, gi = off / VW, kk = (gi >> 6) * VW + off % VW;
      float zt = raw_elem<DT, AL>(ut, 0), zd = raw_elem<DT, AL>(ud, 0);
#pragma unroll
      for (int k = 1; k < 32; ++k) {
        zt = k == kk ? raw_elem<DT, AL>(ut, k) : zt;
        zd = k == kk ? raw_elem<DT, AL>(ud, k) : zd;
      }
      zt = rl_f(zt, gi & 63);
      zd = rl_f(zd, gi & 63);
      const float e1 = __builtin_amdgcn_exp2f(fmaf(zt, s, ot));
      const float e2 = __builtin_amdgcn_exp2f(fmaf(zd, s, od));
      R += fmaxf(fmaf(nkc, e2, e1), 0.f) - fmaxf(fmaf(nk, e2, e1), 0.f);
    }
  }
  return fmaxf(R, 0.f);
}

// Token stage of the bonus drawn from row k*'s residual inside block beta
// (every thread calls; returns the token, -1 if none): r_x = p_x (-expm1(d_x))
// with d_x = ln(c sigma_x) - ln p_x formed in fp64 from the logits (D0 holds
// the constant part), or p_x itself when the row has no residual mass (any =
// false) or the chosen block had mass only through rounding.  Mb: the target
// block maximum of beta; tfl: row k*'s draft top-F list (F entries).
template <int DT, bool AL>
__device__ __forceinline__ int residual_token(const Params& p, int b, const SeqState& ss, int beta, float Mb,
                                              bool any, const int32_t* tfl, uint64_t* slot_r, uint64_t* slot_p) {
  const int tid = threadIdx.x, K1 = p.K + 1, V = (int)p.V, F = p.F;
  const int ks = ss.kstar;
  const int64_t row = (int64_t)b * K1 + ks;
  const int64_t rs = p.ld * Dt<DT>::SZ;
  const unsigned char* rt = p.x + row * rs;
  const unsigned char* rd = p.xd + row * rs;
  const float s = ss.s;
  const int x0 = beta * BLK + TPT * tid;
  Run<DT, AL> runt, rund;
  run_issue<DT, AL>(rt, V, x0, runt);
  run_issue<DT, AL>(rd, V, x0, rund);
  const RaceWords rw = race_words(x0, p.seed, b, ks, ST_BONUS_TOKEN);  // while the blocks load
  __builtin_amdgcn_sched_barrier(0);
  float zt[TPT], zd[TPT];
  run_finish<DT, AL>(V, x0, runt, zt);
  run_finish<DT, AL>(V, x0, rund, zd);
  int x = -1;
  if (any) {
    // r = p - c sigma > 0 iff d = ln(c sigma) - ln p < 0, and then r = p (-expm1(d))
    const uint32_t smask = F <= 0 ? 0u : set_mask(tfl, F, x0);
    const double invT = ss.invT, D0 = ss.D0, lnC = ss.lnC;
    x = token_race(x0, V, rw, slot_r, [&](int e) -> float {
      if (!(zt[e] > -INFINITY)) return INFINITY;
      const float tp = (Mb - zt[e]) * s;
      if (!(zd[e] > -INFINITY)) return tp;
      const double dd = ((double)zd[e] - (double)zt[e]) * invT + D0 + (((smask >> e) & 1u) ? lnC : 0.0);
      if (!(dd < 0.0)) return INFINITY;
      return tp - __builtin_amdgcn_logf(-expm1f((float)dd));
    });
  }
  if (x < 0) {
    x = token_race(x0, V, rw, slot_p, [&](int e) -> float {
      return zt[e] > -INFINITY ? (Mb - zt[e]) * s : INFINITY;
    });
  }
  return x;
}

// Bonus from the residual given its block sums R (thread-owned blocks t +
// k*EWG) and the target row's block maxima Mt (token-tree verification).
template <int DT, bool AL>
__device__ __forceinline__ void epi_residual(const Params& p, int b, const SeqState& ss, const float (&R)[NBT],
                                            const float (&Mt)[NBT], ESm& sm) {
  const int tid = threadIdx.x, K1 = p.K + 1, NB = p.NB, F = p.F;
  const int64_t row = (int64_t)b * K1 + ss.kstar;
  const float s = ss.s, mt = ss.m_t;
#pragma unroll
  for (int k = 0; k < NBT; ++k)
    if (tid + k * EWG < NB) sm.M[tid + k * EWG] = Mt[k];
  const int any = __syncthreads_or(R[0] > 0.f || R[1] > 0.f);
  float M[NBT], S[NBT];
  if (!any) {  // no residual mass: p_k* from the target row's partials
    float4 v[NBT];
#pragma unroll
    for (int k = 0; k < NBT; ++k) v[k] = p.part[row * NB + min(tid + k * EWG, NB - 1)];
#pragma unroll
    for (int k = 0; k < NBT; ++k) {
      const bool in = tid + k * EWG < NB;
      M[k] = in ? v[k].x : -INFINITY;
      S[k] = in ? v[k].y : 0.f;
    }
  }
  int beta = block_stage(NB, p.seed, b, ss.kstar, ST_BONUS_BLOCK, sm.ru[0], [&](int, int k) -> float {
    return any ? R[k] : block_w(M[k], S[k], mt, s);
  });
  if (beta < 0) beta = 0;
  const int32_t* tfl = F > 0 ? p.dtopf + row * p.ld_dtopf : nullptr;
  const int x = residual_token<DT, AL>(p, b, ss, beta, sm.M[beta], any, tfl, sm.ru[1], sm.ru[2]);
  if (tid == 0) {
    p.bonus[b] = (x >= 0 && x < (int)p.V) ? x : 0;
    sm.bonus = (x >= 0 && x < (int)p.V) ? x : 0;
  }
}

// Wave 0's copy of sequence b's keys and payload, one slot per lane, when
// they fit (Bgt <= 64, K <= KREG): fetched at kernel start so the lookup
// needs no load once the bonus is known.
constexpr int KREG = 8;
struct CacheRegs {
  bool ok;
  int key;
  int pay[KREG];
  int fb;  // lane i < K: fallback token i of a miss (when filled), or -1 to draw it at the lookup
};

__device__ __forceinline__ void cache_prefetch(const Params& p, int b, CacheRegs& cr) {
  const int lane = threadIdx.x & 63, K = p.K, Bgt = p.Bgt;
  cr.ok = p.lookup && Bgt <= 64 && K <= KREG;
  cr.key = 0;
  cr.fb = -1;
#pragma unroll
  for (int i = 0; i < KREG; ++i) cr.pay[i] = -1;
  if (!cr.ok || threadIdx.x >= 64 || lane >= Bgt) return;
  const int64_t sl = (int64_t)b * Bgt + lane;
  cr.key = p.ckeys[sl];
#pragma unroll
  for (int i = 0; i < KREG; ++i)
    if (i < K) cr.pay[i] = p.cpay[sl * K + i];
}

// Look (k, y) up among sequence b's keys at depth k (wave 0; every lane
// calls): lowest matching slot, its payload, or a miss.
__device__ __forceinline__ void cache_lookup_wave(const Params& p, int b, int k, int y, const CacheRegs& cr) {
  const int lane = threadIdx.x & 63, K = p.K, Bgt = p.Bgt;
  if (cr.ok) {
    int found = -1;
    if (k >= 0 && k <= K) {
      const uint64_t m = __ballot(lane >= p.koff[k] && lane < p.koff[k + 1] && cr.key == y);
      if (m) found = (int)__builtin_ctzll(m);
    }
    if (lane == 0) {
      p.chit[b] = found >= 0;
      p.cslot[b] = found;
    }
    int t = -1;
    if (found >= 0) {
#pragma unroll
      for (int i = 0; i < KREG; ++i) {
        const int v = __builtin_amdgcn_readlane(cr.pay[i], found);
        t = lane == i ? v : t;
      }
    } else if (p.fill && lane < K) {
      t = cr.fb >= 0 ? cr.fb : fallback_token(p.seed, b, lane, p.V);
    }
    if (lane < K) p.ctok[(int64_t)b * K + lane] = t;
    return;
  }
  int found = -1;
  if (k >= 0 && k <= K) {
    const int lo = p.koff[k], hi = p.koff[k + 1];
    for (int s0 = lo; s0 < hi; s0 += 64) {
      const int sl = s0 + lane;
      const uint64_t m = __ballot(sl < hi && p.ckeys[(int64_t)b * Bgt + min(sl, hi - 1)] == y);
      if (m) {
        found = s0 + __builtin_ctzll(m);
        break;
      }
    }
  }
  if (lane == 0) {
    p.chit[b] = found >= 0;
    p.cslot[b] = found;
  }
  for (int i = lane; i < K; i += 64)
    p.ctok[(int64_t)b * K + i] = found >= 0 ? p.cpay[((int64_t)b * Bgt + found) * K + i]
                                 : p.fill   ? fallback_token(p.seed, b, i, p.V)
                                            : -1;
}

// ---------------------------------------------------------------------------
// Verification of one sequence after its streaming pass (one workgroup):
// statistics of the K + 1 target rows from their partials, the acceptance
// decisions, the bonus and the cache lookup.
//
// The bonus after a rejection at k* is drawn from the residual max(0, p -
// sigma) of row k* by the same two-level race as everywhere (block by its
// residual sum R_be, then a token inside the block), but the block race is
// evaluated lazily: R_be <= P_be, the block's target mass known from the
// streaming partials, so the block key -log2(u_be) / R_be is bounded below
// by -log2(u_be) / P_be.  Blocks are evaluated (both rows re-read, R_be
// summed) smallest bound first, up to LZ_G at a time, until no block left
// has a bound at or below the best exact key: the winner is then the block
// the full race over every R_be would pick, and about 1 / (rejection
// probability) blocks are read instead of two whole rows.  The bound is
// taken with P_be (1 + 1e-3), far above the rounding of either sum.
// ---------------------------------------------------------------------------
constexpr int PM_CAP = 1024;          // per-row block values of the K + 1 rows kept in LDS when (K + 1) NB fits
constexpr int LZ_G = 2 * ENW;         // blocks per round of the lazy block race (two per wave)
constexpr float LZ_INFL = 1.001f;     // R_be <= P_be LZ_INFL
constexpr uint32_t LB_NONE = ~0u;     // no bound: past the row or already evaluated
constexpr uint32_t LB_INF = 0x7F800000u;  // P_be = 0: evaluated only while no block has residual mass
constexpr int LZ_NT = 8;              // steps of the selection ladder

struct VSm {
  uint64_t ru[6][ENW];
  float pM[PM_CAP];         // row j's block be at j NB + be (or only row k* or K, at be)
  float pS[PM_CAP];
  uint32_t lbk[PM_CAP];     // lower bound of row j's block key (the bits of a non-negative float)
  float nlv[PM_CAP];        // -log2(u) of row j's block draw
  int tf[TF_CAP];           // the draft top-F lists of the sequence's rows
  int ckey[64];             // the sequence's cache keys and payload when they fit (CacheRegs)
  int cpay[64 * KREG];
  int cfb[64];              // the fallback tokens of a miss
  int ks;
  SeqState ss;
  float vm[MAX_K1];
  double vL[MAX_K1];
  int vfb[MAX_K1];
  int vam[MAX_K1];
};

// Block bound of the lazy race: -log2(u) / (W LZ_INFL), LB_INF when W = 0.
__device__ __forceinline__ uint32_t lazy_bound(float nl, float W) {
  return W > 0.f ? __float_as_uint(nl * __builtin_amdgcn_rcpf(W * LZ_INFL)) : LB_INF;
}

template <int DT, bool AL, int PLN>
__device__ __forceinline__ void verify_seq(const Params& p, int b, VSm& sm) {
  const int K = p.K, K1 = K + 1, NB = p.NB, tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int V = (int)p.V;
  const int64_t r0 = (int64_t)b * K1;
  const int64_t rs = p.ld * Dt<DT>::SZ;
  // the partials of this wave's first two rows are requested before anything
  // else (every other load and the temperature's would otherwise go first,
  // the temperature's round trip ahead of all of them)
  WRow<PLN> ra, rb;
  load_wrow<PLN>(p.part + (r0 + min(wave, K)) * NB, NB, ra);
  load_wrow<PLN>(p.part + (r0 + min(wave + ENW, K)) * NB, NB, rb);
  // rows of up to 128 blocks (two per lane) keep their block values in LDS
  // when the K + 1 rows fit
  const bool fit = PLN <= 2 && K1 * NB <= PM_CAP;
  SSD_PH_DECL;
  SSD_PH(0);
  // wave 0, lane j < K: drafted token, sigma_j(x_j), the target logit at x_j
  // captured by the streaming pass; lane j <= K: the draft row statistics;
  // thread t < (K+1) F: entry t of the draft top-F lists of all K + 1 rows
  // (the residual of row k* needs one); wave 0: the cache keys and payload.
  // All loaded unconditionally from clamped indices (a valid stand-in array
  // when K = 0 or F = 0: the captured-logit workspace), so that they and the
  // partials above are in flight together (a load under a branch gets a wait
  // of its own) and no load waits on k*.
  const int F = p.F;
  const bool tf_lds = F > 0 && K1 * F <= TF_CAP;
  const int tq = min(tid, max(K - 1, 0));
  const int32_t* dtok = K > 0 ? p.dtok : reinterpret_cast<const int32_t*>(p.zcap);
  const float* dqp = K > 0 ? p.dq : p.zcap;
  const int xl = dtok[b * K + tq];
  const float ql = dqp[b * K + tq], zl = p.zcap[b * K + tq];
  const ssd_row_stats ds = p.dstats[r0 + min(tid, K)];
  const int tt = tf_lds ? min(tid, K1 * F - 1) : 0;
  const int32_t* tfp = tf_lds ? p.dtopf + (r0 + tt / F) * p.ld_dtopf + tt % F : reinterpret_cast<const int32_t*>(p.zcap);
  const int tfv = *tfp;
  CacheRegs cr;
  cache_prefetch(p, b, cr);
  const float T = p.temp[b];
  const bool greedy = !(T > 0.f);
  const float s = greedy ? 0.f : (float)(LOG2E / (double)T);
  const double invT = greedy ? 0.0 : 1.0 / (double)T;
  const int xj = tid < K ? xl : -1;
  const float qj = tid < K ? ql : 0.f, ztj = tid < K ? zl : 0.f;
  const float dmax = (tid <= K && !greedy) ? ds.max : 0.f;
  const double dlse = (tid <= K && !greedy) ? (double)ds.lse : 0.0;
  // row statistics: wave w merges rows j = w, w + ENW, ..., two rows per pass
  // with both rows' loads in flight.  When the rows fit in LDS, their (M, S)
  // stay there with, for rows j < K of T > 0 sequences, the lazy race's
  // block draws (carried by the partials) and bounds.
  const bool pre = fit && !greedy;
  // a row's values after the reductions, kept in LDS
  auto keep = [&](const WRow<PLN>& r, int j, float m, double wsum, const float (&W)[PLN], int fb, int am) {
    if (pre) {
#pragma unroll
      for (int i = 0; i < PLN; ++i) {
        const int be = lane + 64 * i;
        if (be < NB) {
          sm.pM[j * NB + be] = r.M[i];
          sm.pS[j * NB + be] = r.S[i];
          if (j < K) {
            const float nl = __int_as_float(r.I[i]);  // the block draw, from the streaming pass
            sm.lbk[j * NB + be] = lazy_bound(nl, W[i]);
            sm.nlv[j * NB + be] = nl;
          }
        }
      }
    }
    if (lane == 0) {
      sm.vm[j] = m;
      sm.vL[j] = greedy ? 0.0 : ln_fast(wsum);
      sm.vfb[j] = fb < 0 ? 0 : fb;                  // (a NaN row matches no block)
      sm.vam[j] = greedy ? (am < 0 ? 0 : am) : -1;  // greedy rows carry the block argmax in their partial
    }
  };
  // rows ja and jb (jb kept when hb) merged stage by stage, so that the two
  // rows' wave reductions overlap
  auto merge2 = [&](const WRow<PLN>& ra, int ja, const WRow<PLN>& rb, int jb, bool hb) {
    float la = ra.M[0], lb = rb.M[0];
#pragma unroll
    for (int i = 1; i < PLN; ++i) {
      la = fmaxf(la, ra.M[i]);
      lb = fmaxf(lb, rb.M[i]);
    }
    const float ma = wave_max(la), mb = wave_max(lb);
    int fba = -1, ama = -1, fbb = -1, amb = -1;
    double sa = 0.0, sb = 0.0;
    float Wa[PLN], Wb[PLN];
#pragma unroll
    for (int i = PLN - 1; i >= 0; --i) {
      Wa[i] = greedy ? 0.f : block_w(ra.M[i], ra.S[i], ma, s);
      Wb[i] = greedy ? 0.f : block_w(rb.M[i], rb.S[i], mb, s);
      sa += (double)Wa[i];
      sb += (double)Wb[i];
      const uint64_t ka = __ballot(lane + 64 * i < NB && ra.M[i] == ma);
      const uint64_t kb = __ballot(lane + 64 * i < NB && rb.M[i] == mb);
      if (ka) {
        fba = 64 * i + (int)__builtin_ctzll(ka);
        ama = __builtin_amdgcn_readlane(ra.I[i], (int)__builtin_ctzll(ka));
      }
      if (kb) {
        fbb = 64 * i + (int)__builtin_ctzll(kb);
        amb = __builtin_amdgcn_readlane(rb.I[i], (int)__builtin_ctzll(kb));
      }
    }
    sa = wave_sum_d(sa);
    sb = wave_sum_d(sb);
    keep(ra, ja, ma, sa, Wa, fba, ama);
    if (hb) keep(rb, jb, mb, sb, Wb, fbb, amb);
  };
  float uacc = 0.f;
  int fbt = -1;
  for (int j0 = wave; j0 < K1; j0 += 2 * ENW) {
    const int j1 = j0 + ENW;
    if (j0 != wave) {  // (K + 1 > 2 ENW rows only)
      load_wrow<PLN>(p.part + (r0 + j0) * NB, NB, ra);
      load_wrow<PLN>(p.part + (r0 + min(j1, K)) * NB, NB, rb);
    }
    // wave 0, lane j: the acceptance draw u_j and the fallback token j of a
    // cache miss, computed while the partials load
    if (wave == 0 && j0 == 0) {
      if (!greedy) uacc = uniform_of(draw1(p.seed, 0u, (uint32_t)b, (uint32_t)lane, ST_ACCEPT));
      if (cr.ok && p.fill && lane < K) fbt = fallback_token(p.seed, b, lane, p.V);
    }
    merge2(ra, j0, rb, j1, j1 < K1);
  }
  if (tf_lds && tid < K1 * F) sm.tf[tid] = tfv;
  // the cache keys and payload wait in LDS (registers are short later on),
  // with the fallback tokens of a miss (drawn while the partials loaded)
  if (cr.ok && tid < 64) {
    sm.ckey[lane] = cr.key;
#pragma unroll
    for (int i = 0; i < KREG; ++i) sm.cpay[lane * KREG + i] = cr.pay[i];
    sm.cfb[lane] = fbt;
  }
  lds_sync();
  SSD_PH(1);  // prologue loads and the K+1 rows' statistics
  // argmax of the T > 0 rows is only needed for the optional statistics
  if (!greedy && p.stats) {
    for (int j = wave; j < K1; j += ENW) {
      const int am = wave_first_eq<DT, AL>(p.x + (r0 + j) * rs, V, sm.vfb[j], sm.vm[j]);
      if (lane == 0) sm.vam[j] = am;
    }
    lds_sync();
  }
  // acceptance decisions (wave 0, lane j < K) and p_j(x_j) for every position
  double pj = 0.0;
  if (wave == 0) {
    bool acc = false;
    if (lane < K && xj >= 0 && xj < V) {
      if (greedy) {
        acc = (xj == sm.vam[lane]);
        pj = acc ? 1.0 : 0.0;
      } else {
        pj = exp_fast(((double)ztj - (double)sm.vm[lane]) * invT - sm.vL[lane]);
        // u < p / q taken as u q < p (q > 0): the two differ only where u
        // and p / q agree to the last bits of fp64, a near tie
        const double q = (double)qj;
        acc = q > 0.0 ? (double)uacc * q < pj : pj > 0.0;
      }
    }
    const uint64_t rej = __ballot(lane < K && !acc);
    const int ks = rej ? (int)__builtin_ctzll(rej) : K;
    SeqState ss{};
    ss.kstar = ks;
    if (!greedy && ks < K) {
      // the residual's constants (target and draft row k*)
      const float mt = sm.vm[ks];
      const float md = rl_f(dmax, ks);
      const double Ld = rl_d(dlse, ks), Lt = sm.vL[ks];
      ss.need = 1;
      ss.s = s;
      ss.m_t = mt;
      ss.o_t = -mt * s;
      ss.o_d = -md * s;
      const double et = (double)ss.o_t + (double)mt * (double)s;
      const double ed = (double)ss.o_d + (double)md * (double)s;
      ss.invT = invT;
      ss.D0 = ((double)mt - (double)md) * invT + Lt - Ld;
      ss.lnC = ln_fast((double)p.C);
      ss.kf = (float)exp_fast((et - ed) * LN2 + (Lt - Ld));
    }
    if (lane == 0) {
      sm.ks = ks;
      sm.ss = ss;
    }
  }
  lds_sync();
  SSD_PH(2);  // acceptance decisions
  const int ks = sm.ks;
  const float pjf = (float)pj;
  int y = greedy ? sm.vam[ks] : 0;  // the bonus
  if (!greedy) {
    // row k*'s partials (row K when every token is accepted): kept by the
    // merge, or read again now
    int pb = ks * NB;
    if (!fit) {
      for (int be = tid; be < NB; be += EWG) {
        const float4 v = p.part[(r0 + ks) * NB + be];
        sm.pM[be] = v.x;
        sm.pS[be] = v.y;
        sm.nlv[be] = v.z;
      }
      lds_sync();
      pb = 0;
    }
    int x;
    if (ks == K) {
      // all K accepted: bonus ~ p_K
      const float m = sm.vm[K];
      int beta = block_stage(NB, p.seed, b, K, ST_BONUS_BLOCK, sm.ru[0], [&](int be, int) -> float {
        return block_w(sm.pM[pb + be], sm.pS[pb + be], m, s);
      });
      if (beta < 0) beta = 0;
      const unsigned char* rp = p.x + (r0 + K) * rs;
      const int x0 = beta * BLK + TPT * tid;
      Run<DT, AL> run;
      run_issue<DT, AL>(rp, V, x0, run);
      const RaceWords rw = race_words(x0, p.seed, b, K, ST_BONUS_TOKEN);  // while the block loads
      __builtin_amdgcn_sched_barrier(0);
      float z[TPT];
      run_finish<DT, AL>(V, x0, run, z);
      const float Mb = sm.pM[pb + beta];
      x = token_race(x0, V, rw, sm.ru[1], [&](int e) -> float {
        return z[e] > -INFINITY ? (Mb - z[e]) * s : INFINITY;
      });
      SSD_PH(3);
    } else {
      // lazy block race over the residual of row k*
      const SeqState ss = sm.ss;
      const int64_t row = r0 + ks;
      const unsigned char* rt = p.x + row * rs;
      const unsigned char* rd = p.xd + row * rs;
      const int32_t* tfl = F <= 0 ? nullptr : tf_lds ? sm.tf + ks * F : p.dtopf + row * p.ld_dtopf;
      const float ot = ss.o_t, od = ss.o_d, nk = -ss.kf, nkc = nk * p.C, mt = ss.m_t;
      // every wave holds every block's bound (block be = lane + 64 i in slot i)
      uint32_t lb[PLN];
      float nl[PLN];
#pragma unroll
      for (int i = 0; i < PLN; ++i) {
        const int be = lane + 64 * i;
        const bool in = be < NB;
        if (fit) {
          lb[i] = in ? sm.lbk[pb + be] : LB_NONE;
          nl[i] = in ? sm.nlv[pb + be] : 0.f;
        } else {
          const float W = in ? block_w(sm.pM[pb + be], sm.pS[pb + be], mt, s) : 0.f;
          nl[i] = in ? sm.nlv[pb + be] : 0.f;
          lb[i] = in ? lazy_bound(nl[i], W) : LB_NONE;
        }
      }
      uint64_t best = NO_KEY;
      int nev = 0;
      for (int round = 0;; ++round) {
        // the candidates: bounds at or below the best key so far.  A round
        // takes those up to m c_t (m: the smallest; c_t: the ladder's largest
        // step that keeps them within LZ_G), or the first LZ_G of the ties at
        // m; the same choice in every wave.
        const uint32_t lim = (uint32_t)(best >> 32);
        uint32_t mn = lb[0];
#pragma unroll
        for (int i = 1; i < PLN; ++i) mn = min(mn, lb[i]);
        mn = wave_min_u32(mn);
        if (mn == LB_NONE || mn > lim) break;
        constexpr float ladder[LZ_NT] = {1.f, 1.5f, 2.f, 3.f, 4.f, 8.f, 16.f, 64.f};
        const float mf = __uint_as_float(mn);
        uint32_t thr = mn;
#pragma unroll
        for (int t = 1; t < LZ_NT; ++t) {
          const uint32_t tb = min(__float_as_uint(mf * ladder[t]), lim);
          int cnt = 0;
#pragma unroll
          for (int i = 0; i < PLN; ++i) cnt += __popcll(__ballot(lb[i] <= tb));
          thr = cnt <= LZ_G ? tb : thr;
        }
        // the chosen blocks (the first LZ_G at or below the threshold, in
        // increasing index), two per wave; every wave marks all of them
        // evaluated
        int sel0 = -1, sel1 = -1, nsel = 0;
#pragma unroll
        for (int i = 0; i < PLN; ++i) {
          const uint64_t m0 = __ballot(lb[i] <= thr);
          uint64_t mk = m0;
          while (mk && nsel < LZ_G) {
            const int be = 64 * i + (int)__builtin_ctzll(mk);
            mk &= mk - 1ull;
            sel0 = nsel == wave ? be : sel0;
            sel1 = nsel == wave + ENW ? be : sel1;
            ++nsel;
          }
          lb[i] = ((m0 ^ mk) >> lane) & 1ull ? LB_NONE : lb[i];
        }
        float n0 = 0.f, n1 = 0.f;
        if (sel0 >= 0) n0 = slot_at<PLN>(nl, sel0);
        if (sel1 >= 0) n1 = slot_at<PLN>(nl, sel1);
        nev += nsel;
        uint64_t wb = NO_KEY;
        if (sel0 >= 0) {
          const int c1 = sel1 >= 0 ? sel1 : sel0;
          RawBlock<DT, AL> ut0, ud0, ut1, ud1;
          // ordinary loads: the chosen block is read again by the token stage
          if ((max(sel0, c1) + 1) * BLK <= V) {
            load_raw<DT, AL, true, false>(rt, V, sel0, lane, ut0);
            load_raw<DT, AL, true, false>(rd, V, sel0, lane, ud0);
            load_raw<DT, AL, true, false>(rt, V, c1, lane, ut1);
            load_raw<DT, AL, true, false>(rd, V, c1, lane, ud1);
          } else {
            load_raw<DT, AL, false>(rt, V, sel0, lane, ut0);
            load_raw<DT, AL, false>(rd, V, sel0, lane, ud0);
            load_raw<DT, AL, false>(rt, V, c1, lane, ut1);
            load_raw<DT, AL, false>(rd, V, c1, lane, ud1);
          }
          const float R0 = block_residual<DT, AL>(ut0, ud0, sel0, V, s, ot, od, nk, nkc, F, tfl);
          if (R0 > 0.f) wb = race_key(n0 * __builtin_amdgcn_rcpf(R0), sel0);
          if (sel1 >= 0) {
            const float R1 = block_residual<DT, AL>(ut1, ud1, sel1, V, s, ot, od, nk, nkc, F, tfl);
            if (R1 > 0.f) wb = umin64(wb, race_key(n1 * __builtin_amdgcn_rcpf(R1), sel1));
          }
        }
        // (two alternating slots: a wave rewrites one only after the next
        // barrier, which every wave reaches after reading it)
        uint64_t* slot = sm.ru[2 + (round & 1)];
        if (lane == 0) slot[wave] = wb;
        lds_sync();
#pragma unroll
        for (int w = 0; w < ENW; ++w) best = umin64(best, slot[w]);
      }
      SSD_PH(3);  // lazy block race
      SSD_PH_SET(7, nev);
      (void)nev;
      const bool any = best != NO_KEY;
      int beta = (int)(uint32_t)best;
      if (!any) {
        // no residual mass (every block evaluated): p_k*
        beta = block_stage(NB, p.seed, b, ks, ST_BONUS_BLOCK, sm.ru[0], [&](int be, int) -> float {
          return block_w(sm.pM[pb + be], sm.pS[pb + be], mt, s);
        });
        if (beta < 0) beta = 0;
      }
      x = residual_token<DT, AL>(p, b, ss, beta, sm.pM[pb + beta], any, tfl, sm.ru[1], sm.ru[4]);
    }
    y = (x >= 0 && x < V) ? x : 0;
  }
  SSD_PH(4);  // bonus token
  if (p.lookup && tid < 64) {
    CacheRegs c2;
    c2.ok = cr.ok;
    c2.key = cr.ok ? sm.ckey[lane] : 0;
    c2.fb = cr.ok ? sm.cfb[lane] : -1;
#pragma unroll
    for (int i = 0; i < KREG; ++i) c2.pay[i] = cr.ok ? sm.cpay[lane * KREG + i] : -1;
    cache_lookup_wave(p, b, ks, y, c2);
  }
  SSD_PH(5);  // cache lookup
  // the per-sequence outputs, stored last: a barrier, or a wait for an older
  // load, after a store waits for the store too (one counter covers both)
  if (wave == 0) {
    // (early exit: the rows past k* may not have been read)
    if (lane < K) p.p_out[b * K + lane] = (p.early && lane > ks) ? __builtin_nanf("") : pjf;
    if (lane == 0) {
      p.acc_len[b] = ks;
      p.bonus[b] = y;
    }
  }
  if (p.stats && tid < K1) {
    ssd_row_stats st;
    st.lse = sm.vL[tid];
    st.max = sm.vm[tid];
    st.argmax = sm.vam[tid];
    p.stats[r0 + tid] = st;
  }
  SSD_PH_FLUSH(1, b);
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------
// (f32 and unaligned rows need more registers per element: fewer waves)
template <int DT, bool AL, int MODE>
__device__ __forceinline__ void stream_item(const Params& p, int item) {
  const int64_t it = item / p.nchunk;
  const int chunk = item - (int)(it * p.nchunk);
  const int64_t row = p.jn > 0 ? (it / p.jn) * (p.K + 1) + p.jlo + (it % p.jn) : it;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K1 = p.K + 1;
  const unsigned char* rp = p.x + row * p.ld * Dt<DT>::SZ;
  const int V = (int)p.V, NB = p.NB;
  const int b0 = chunk * CH + wave, b1 = b0 + NWAVE;
  // the logit loads are issued first; the temperature (and the drafted
  // token) are fetched behind them
  RawBlock<DT, AL> r0, r1;
  const bool full = (chunk + 1) * CH * BLK <= V;
  // verification: the first p.keep target rows of a sequence, the likeliest
  // rows of the first rejection, are read with ordinary loads so that the
  // residual pass's re-read of row k* may find them in the Infinity Cache
  const bool keep = MODE == M_VERIFY && (int)(row % K1) < p.keep;
  if (full && keep) {
    load_raw<DT, AL, true, false>(rp, V, b0, lane, r0);
    load_raw<DT, AL, true, false>(rp, V, b1, lane, r1);
  } else if (full) {
    // every block of this chunk is full: all loads in flight together
    load_raw<DT, AL, true>(rp, V, b0, lane, r0);
    load_raw<DT, AL, true>(rp, V, b1, lane, r1);
  } else {
    // the chunk holding the ragged end of the row
    load_raw<DT, AL, false>(rp, V, min(b0, NB - 1), lane, r0);
    load_raw<DT, AL, false>(rp, V, min(b1, NB - 1), lane, r1);
  }
  float T = 0.f;
  if constexpr (MODE == M_SOFTMAX) T = p.temp[row];
  if constexpr (MODE == M_SAMPLE || MODE == M_VERIFY) T = p.temp[row / K1];
  const double sd = LOG2E / (double)T;
  const float s = (T > 0.f) ? (float)sd : 0.f;
  int xj = -1;  // verification: drafted token of this target row (j < K)
  if constexpr (MODE == M_VERIFY) {
    const int j = (int)(row % K1);
    if (j < p.K && p.dtok) xj = p.dtok[(row / K1) * p.K + j];
  }
  float v[32];
  decode_raw<DT, AL>(r0, v);
  float4 P0 = block_partial<DT, MODE>(v, s, min(b0, NB - 1), lane);
  decode_raw<DT, AL>(r1, v);
  float4 P1 = block_partial<DT, MODE>(v, s, min(b1, NB - 1), lane);
  if constexpr (MODE == M_VERIFY) {
    // T > 0 rows leave I unused: it carries -log2(u) of the block's draw for
    // a bonus from this row, u(idx = block, b, j, bonus-block stream), which
    // the verification's lazy block race reads with the partials (the
    // counters are uniform in the workgroup: scalar arithmetic)
    if (s > 0.f) {
      const uint32_t bq = (uint32_t)(row / K1), jq = (uint32_t)(row % K1);
      P0.z = neg_log2_u(draw1(p.seed, (uint32_t)b0, bq, jq, ST_BONUS_BLOCK));
      P1.z = neg_log2_u(draw1(p.seed, (uint32_t)b1, bq, jq, ST_BONUS_BLOCK));
    }
  }
  if (lane == 0 && b0 < NB) p.part[row * NB + b0] = P0;
  if (lane == 0 && b1 < NB) p.part[row * NB + b1] = P1;
  if constexpr (MODE == M_VERIFY) {
    if (p.gate_reset && item == 0 && threadIdx.x == 0) p.gate[0] = 0;
  }
  if constexpr (MODE == M_VERIFY) {
    // the workgroup whose chunk holds x_j hands its target logit to the epilogue
    if (xj >= 0 && xj < V && xj / (CH * BLK) == chunk && threadIdx.x == 0)
      p.zcap[(row / K1) * p.K + (row % K1)] = load_elem<DT>(rp, xj);
  }
}

template <int DT, bool AL, int MODE>
__global__ __launch_bounds__(WG, (DT == SSD_F32 || !AL) ? 4 : 6) void k_stream(Params p) {
  stream_item<DT, AL, MODE>(p, blockIdx.x);
}

// Early-exit verification.  A sequence's verification never reads target
// rows past its first rejection, so once positions 0 .. J-1 have been
// streamed, the rows from J on are needed only by sequences without a
// rejection below J.  seq_alive judges that from the partials of rows < J
// (written by the previous launch) conservatively: false only when some
// position j < J is rejected with a clear margin (T > 0: u_j >= rho_j (1 +
// 1e-4); greedy: x_j is not the row's argmax; or x_j outside [0, V)), so a
// sequence that the acceptance pass may find unrejected below J is never
// skipped.  Every thread calls; the result is uniform.
struct GateSm {
  float m[MAX_K1];
  double L[MAX_K1];
  int am[MAX_K1];
  int alive;
};
template <int PLN>
__device__ __forceinline__ bool seq_alive(const Params& p, int b, int J, GateSm& g) {
  const int K = p.K, K1 = K + 1, NB = p.NB, V = (int)p.V;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float T = p.temp[b];
  const bool greedy = !(T > 0.f);
  const float s = greedy ? 0.f : (float)(LOG2E / (double)T);
  const int Jd = min(J, K);  // positions with a decision
  for (int j = wave; j < Jd; j += NWAVE) {
    WRow<PLN> r;
    load_wrow<PLN>(p.part + ((int64_t)b * K1 + j) * NB, NB, r);
    float lm = r.M[0];
#pragma unroll
    for (int i = 1; i < PLN; ++i) lm = fmaxf(lm, r.M[i]);
    const float m = wave_max(lm);
    double ws = 0.0;
    int am = -1;
#pragma unroll
    for (int i = PLN - 1; i >= 0; --i) {
      if (!greedy) ws += (double)block_w(r.M[i], r.S[i], m, s);
      const uint64_t mk = __ballot(lane + 64 * i < NB && r.M[i] == m);
      if (mk) am = __builtin_amdgcn_readlane(r.I[i], (int)__builtin_ctzll(mk));
    }
    ws = wave_sum_d(ws);
    if (lane == 0) {
      g.m[j] = m;
      g.L[j] = greedy ? 0.0 : ln_fast(ws);
      g.am[j] = am < 0 ? 0 : am;
    }
  }
  lds_sync();
  if (wave == 0) {
    bool rej = false;
    if (lane < Jd) {
      const int xj = p.dtok[b * K + lane];
      if (xj < 0 || xj >= V) {
        rej = true;
      } else if (greedy) {
        rej = xj != g.am[lane];
      } else {
        const double pj = exp_fast(((double)p.zcap[b * K + lane] - (double)g.m[lane]) * (1.0 / (double)T) - g.L[lane]);
        const double q = (double)p.dq[b * K + lane];
        const double rho = q > 0.0 ? pj / q : (pj > 0.0 ? INFINITY : 0.0);
        const double u = (double)uniform_of(draw1(p.seed, 0u, (uint32_t)b, (uint32_t)lane, ST_ACCEPT));
        rej = u >= rho * (1.0 + 1e-4) + 1e-30;
      }
    }
    const uint64_t rm = __ballot(rej);
    if (lane == 0) g.alive = rm == 0ull;
  }
  lds_sync();
  return g.alive != 0;
}

// The early-exit gate, decided once per sequence (one workgroup each) over
// the partials of positions 0 .. jlo - 1: a kept sequence takes the next
// place of the list (its order follows the atomics, which changes only which
// workgroup streams which rows).
template <int DT, bool AL>
__global__ __launch_bounds__(EWG) void k_gate(Params p) {
  __shared__ GateSm g;
  const int b = blockIdx.x;
  const bool alive = p.NB <= 128 ? seq_alive<2>(p, b, p.jlo, g) : seq_alive<NBL>(p, b, p.jlo, g);
  if (alive && threadIdx.x == 0) p.gate[1 + atomicAdd(&p.gate[0], 1)] = b;
}

// Streaming pass of verification over positions jlo .. jlo + jn - 1 of the
// sequences the gate kept: workgroup g streams item g % per of the
// (g / per)-th listed sequence; workgroups past the list return (they come
// last, so the kept rows fill the machine first).
template <int DT, bool AL>
__global__ __launch_bounds__(WG, (DT == SSD_F32 || !AL) ? 4 : 6) void k_stream_gated(Params p) {
  const int per = p.jn * p.nchunk;
  const int k = (int)blockIdx.x / per;
  const int n = p.gate[0], b = p.gate[1 + k];  // (both loads issued together; k < B)
  if (k >= n) return;
  stream_item<DT, AL, M_VERIFY>(p, b * per + (int)blockIdx.x % per);
}

// Sampling epilogue item g: row g, or (g >= rows) a long cache-key list.
template <int DT, bool AL>
__device__ __forceinline__ void sample_epi_item(const Params& p, int g, ESm& sm) {
  const bool small = p.NB <= 128;
  if (g < p.rows) small ? epi_sample_p<DT, AL, 2>(p, g, sm) : epi_sample_p<DT, AL, NBL>(p, g, sm);
  else small ? epi_keys_p<DT, AL, 2>(p, g - (int)p.rows, sm) : epi_keys_p<DT, AL, NBL>(p, g - (int)p.rows, sm);
}

// One workgroup per row (per sequence for verification) over the partials.
template <int DT, bool AL, int MODE>
__global__ __launch_bounds__(EWG) void k_epi(Params p) {
  __shared__ ESm sm;
  const int g = blockIdx.x;
  // rows of up to 128 blocks (V <= 262144) keep two partials per lane
  const bool small = p.NB <= 128;
  if constexpr (MODE == M_SOFTMAX) small ? epi_softmax_p<DT, AL, 2>(p, g) : epi_softmax_p<DT, AL, NBL>(p, g);
  if constexpr (MODE == M_TOPF) small ? epi_topf_p<DT, AL, 2>(p, g, sm) : epi_topf_p<DT, AL, NBL>(p, g, sm);
  if constexpr (MODE == M_SAMPLE) sample_epi_item<DT, AL>(p, g, sm);
}

// Verification after the streaming pass: one workgroup per sequence.
template <int DT, bool AL>
__device__ __forceinline__ void verify_item(const Params& p, int b, VSm& sm) {
  if (p.NB <= 128) verify_seq<DT, AL, 2>(p, b, sm);
  else verify_seq<DT, AL, NBL>(p, b, sm);
}

template <int DT, bool AL>
__global__ __launch_bounds__(EWG) void k_verify_seq(Params p) {
  __shared__ VSm sm;
  verify_item<DT, AL>(p, blockIdx.x, sm);
}

// One round of the pipeline: the verification of round i (one workgroup per
// sequence, below nv) beside the streaming pass of round i + 1's sampling,
// which does not depend on it.
template <int DT, bool AL>
__global__ __launch_bounds__(EWG, (DT == SSD_F32 || !AL) ? 3 : 4) void k_round_mid(Params pv, Params ps, int nv) {
  __shared__ VSm sm;
  if ((int)blockIdx.x < nv) verify_item<DT, AL>(pv, blockIdx.x, sm);
  else stream_item<DT, AL, M_SAMPLE>(ps, (int)blockIdx.x - nv);
}

// Small batches: a round in two launches instead, (1) both streaming passes
// (round i's target rows, below nv; round i + 1's draft rows), (2) the
// verification of each sequence of round i beside round i + 1's sampling
// epilogue (below nv: the verification).
template <int DT, bool AL>
__global__ __launch_bounds__(WG, (DT == SSD_F32 || !AL) ? 4 : 6) void k_round_streams(Params pv, Params ps, int nv) {
  if ((int)blockIdx.x < nv) stream_item<DT, AL, M_VERIFY>(pv, blockIdx.x);
  else stream_item<DT, AL, M_SAMPLE>(ps, (int)blockIdx.x - nv);
}

union TailSm {
  VSm v;
  ESm e;
};
template <int DT, bool AL>
__global__ __launch_bounds__(EWG) void k_round_tails(Params pv, Params ps, int nv) {
  __shared__ TailSm sm;
  if ((int)blockIdx.x < nv) verify_item<DT, AL>(pv, blockIdx.x, sm.v);
  else sample_epi_item<DT, AL>(ps, (int)blockIdx.x - nv, sm.e);
}

// ---------------------------------------------------------------------------
// Token-tree verification: recursive rejection sampling over the drafted
// children of each node (the residual renormalised after each rejected
// sibling).  After m rejections at node n the residual is max(0, p - c sigma)
// / N with scalars c and N: starting from c = 0, N = 1 (r = p), a rejection
// sets c <- c + N and N <- sum_x max(0, p_x - c sigma_x), one pass over the
// node's target and draft rows (kept when it has mass, as a residual without
// mass leaves r unchanged).  One workgroup per sequence walks the tree from
// the root; every wave takes the same decisions on its own copy of the
// per-node values (one lane per node), and the passes split the blocks over
// the waves.
// ---------------------------------------------------------------------------
constexpr int MAX_TN = 64;  // tree nodes (root included)

struct TreeArgs {
  uint64_t par[MAX_TN / 8];  // parent of node m in byte m (the root's is unused)
  int N1;                    // nodes, root included
  int32_t* last;             // out: node where the walk stopped [B]
};

struct TreeSm {
  float vm[MAX_TN];
  double vL[MAX_TN];
  int vam[MAX_TN];
  float R[2][MAX_NB];   // residual block sums of the current and previous pass
  double rsum[ENW];
};

__device__ __forceinline__ int tree_parent(const TreeArgs& ta, int m) {
  uint64_t w = ta.par[0];
#pragma unroll
  for (int i = 1; i < MAX_TN / 8; ++i) w = ((m >> 3) == i) ? ta.par[i] : w;
  return (int)((w >> (8 * (m & 7))) & 0xFFu);
}

template <int DT, bool AL, int PLN>
__device__ __forceinline__ void tree_item(const Params& p, const TreeArgs& ta, int b, ESm& sm, TreeSm& ts) {
  const int N1 = ta.N1, NB = p.NB, V = (int)p.V, F = p.F, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const float T = p.temp[b];
  const bool greedy = !(T > 0.f);
  const float s = greedy ? 0.f : (float)(LOG2E / (double)T);
  const double invT = greedy ? 0.0 : 1.0 / (double)T;
  const int64_t r0 = (int64_t)b * N1;
  const int64_t rs = p.ld * Dt<DT>::SZ;
  // lane m: node m's parent, token, sigma_parent(token), the target logit at
  // the token (row of the parent) and its own draft row statistics
  const bool node = lane < N1;
  const int nm = node ? lane : 0;
  const int par = (node && lane > 0) ? tree_parent(ta, lane) : -1;
  const int tok = (node && lane > 0) ? p.dtok[r0 + nm] : -1;
  const float qv = (node && lane > 0) ? p.dq[r0 + nm] : 0.f;
  const ssd_row_stats dsn = p.dstats[r0 + nm];
  const bool tin = tok >= 0 && tok < V;
  const float zc = tin ? load_elem<DT>(p.x + (r0 + par) * rs, tok) : 0.f;
  // row statistics of every node from the streaming partials, two rows per
  // wave and pass
  for (int j0 = wave; j0 < N1; j0 += 2 * ENW) {
    const int j1 = j0 + ENW;
    WRow<PLN> ra, rb;
    load_wrow<PLN>(p.part + (r0 + j0) * NB, NB, ra);
    load_wrow<PLN>(p.part + (r0 + min(j1, N1 - 1)) * NB, NB, rb);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const WRow<PLN>& r = h ? rb : ra;
      const int j = h ? j1 : j0;
      if (j >= N1) break;
      float lm = r.M[0];
#pragma unroll
      for (int i = 1; i < PLN; ++i) lm = fmaxf(lm, r.M[i]);
      const float m = wave_max(lm);
      int am = -1;
      double wsum = 0.0;
#pragma unroll
      for (int i = PLN - 1; i >= 0; --i) {
        if (!greedy) wsum += (double)block_w(r.M[i], r.S[i], m, s);
        const uint64_t mk = __ballot(lane + 64 * i < NB && r.M[i] == m);
        if (mk) am = __builtin_amdgcn_readlane(r.I[i], (int)__builtin_ctzll(mk));
      }
      wsum = wave_sum_d(wsum);
      if (lane == 0) {
        ts.vm[j] = m;
        ts.vL[j] = greedy ? 0.0 : ln_fast(wsum);
        ts.vam[j] = am < 0 ? 0 : am;
      }
    }
  }
  lds_sync();
  int n = 0, depth = 0, cur = 0;
  double c = 0.0, Nr = 1.0;  // residual max(0, p - c sigma) / Nr at node n
  bool res = false;          // the bonus comes from a residual with mass
  for (;;) {
    // the residual state belongs to the node the walk is at
    c = 0.0;
    Nr = 1.0;
    res = false;
    const uint64_t kids = __ballot(node && lane > 0 && par == n);
    if (greedy) {
      const uint64_t ok = __ballot(node && lane > 0 && par == n && tok == ts.vam[n]);
      if (!ok) break;
      n = (int)__builtin_ctzll(ok);
      ++depth;
      continue;
    }
    if (!kids) break;
    const float mt = ts.vm[n];
    const double Lt = ts.vL[n];
    int next = -1;
    uint64_t km = kids;
    for (int i = 0; km; ++i) {
      const int m = (int)__builtin_ctzll(km);
      km &= km - 1ull;
      const int x = __builtin_amdgcn_readlane(tok, m);
      const double q = (double)rl_f(qv, m);
      const double px = (x >= 0 && x < V) ? exp_fast(((double)rl_f(zc, m) - (double)mt) * invT - Lt) : 0.0;
      const double num = px - c * q;
      double rho;
      if (!(x >= 0 && x < V)) rho = 0.0;
      else if (q > 0.0) rho = fmax(num, 0.0) / (Nr * q);
      else rho = px > 0.0 ? INFINITY : 0.0;
      const double u = (double)uniform_of(draw1(p.seed, (uint32_t)i, (uint32_t)b, (uint32_t)n, ST_ACCEPT));
      if (u < rho) {
        next = m;
        break;
      }
      // rejected: the residual with c' = c + Nr, summed per block into R[nxt]
      const double cn = c + Nr;
      const int nxt = cur ^ 1;
      const float md = rl_f(dsn.max, n);
      const double Ld = rl_d(dsn.lse, n);
      const float ot = -mt * s, od = -md * s;
      const double et = (double)ot + (double)mt * (double)s, ed = (double)od + (double)md * (double)s;
      const float kf = (float)exp_fast((et - ed) * LN2 + (Lt - Ld));
      const float nk = -(float)(cn * (double)kf), nkc = nk * p.C;
      const int64_t row = r0 + n;
      const unsigned char* rt = p.x + row * rs;
      const unsigned char* rd = p.xd + row * rs;
      const int32_t* tfrow = F > 0 ? p.dtopf + row * p.ld_dtopf : nullptr;
      if (tid < F) sm.tf[tid] = tfrow[tid];
      lds_sync();
      double wacc = 0.0;
      for (int base = 0; base < NB; base += CH_R) {
        const int be0 = base + wave, be1 = be0 + ENW;
        if (be0 >= NB) break;
        RawBlock<DT, AL> ut0, ud0, ut1, ud1;
        if ((base + CH_R) * BLK <= V) {
          load_raw<DT, AL, true>(rt, V, be0, lane, ut0);
          load_raw<DT, AL, true>(rd, V, be0, lane, ud0);
          load_raw<DT, AL, true>(rt, V, be1, lane, ut1);
          load_raw<DT, AL, true>(rd, V, be1, lane, ud1);
        } else {
          load_raw<DT, AL, false>(rt, V, be0, lane, ut0);
          load_raw<DT, AL, false>(rd, V, be0, lane, ud0);
          load_raw<DT, AL, false>(rt, V, min(be1, NB - 1), lane, ut1);
          load_raw<DT, AL, false>(rd, V, min(be1, NB - 1), lane, ud1);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int be = h ? be1 : be0;
          if (be >= NB) break;
          const RawBlock<DT, AL>& ut = h ? ut1 : ut0;
          const RawBlock<DT, AL>& ud = h ? ud1 : ud0;
          const float R = block_residual<DT, AL>(ut, ud, be, V, s, ot, od, nk, nkc, F, sm.tf);
          if (lane == 0) ts.R[nxt][be] = R;
          wacc += (double)R;
        }
      }
      if (lane == 0) ts.rsum[wave] = wacc;
      lds_sync();
      double tot = 0.0;
#pragma unroll
      for (int w = 0; w < ENW; ++w) tot += ts.rsum[w];
      // back to probability units: p_x = e1 2^(-et) e^(-Lt)
      const double Nn = tot * exp_fast(-et * LN2 - Lt);
      if (Nn > 0.0) {
        c = cn;
        Nr = Nn;
        cur = nxt;
        res = true;
      }
      lds_sync();  // (the next pass rewrites the other buffer and the top-F list)
    }
    if (next < 0) break;
    n = next;
    ++depth;
  }
  if (tid == 0) {
    p.acc_len[b] = depth;
    ta.last[b] = n;
    if (greedy) p.bonus[b] = ts.vam[n];
  }
  if (greedy) return;
  // bonus at node n: from the residual of the last pass with mass, else
  // from p_n (a leaf, or no rejection left any residual mass)
  SeqState ss{};
  ss.kstar = n;
  ss.s = s;
  ss.m_t = ts.vm[n];
  ss.invT = invT;
  const float md = rl_f(dsn.max, n);
  const double Ld = rl_d(dsn.lse, n);
  ss.D0 = ((double)ss.m_t - (double)md) * invT + ts.vL[n] - Ld + (res ? ln_fast(c) : 0.0);
  ss.lnC = ln_fast((double)p.C);
  float R[NBT], Mt[NBT];
  const float4* tp = p.part + (r0 + n) * NB;
#pragma unroll
  for (int k = 0; k < NBT; ++k) {
    const int be = tid + k * EWG;
    const bool in = be < NB;
    Mt[k] = in ? tp[min(be, NB - 1)].x : -INFINITY;
    R[k] = (in && res) ? ts.R[cur][be] : 0.f;
  }
  epi_residual<DT, AL>(p, b, ss, R, Mt, sm);
}

template <int DT, bool AL>
__global__ __launch_bounds__(EWG) void k_tree(Params p, TreeArgs ta) {
  __shared__ ESm sm;
  __shared__ TreeSm ts;
  if (p.NB <= 128) tree_item<DT, AL, 2>(p, ta, blockIdx.x, sm, ts);
  else tree_item<DT, AL, NBL>(p, ta, blockIdx.x, sm, ts);
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

// One wave per sequence: find the bonus among depth k*'s keys (lowest slot).
// The depth offsets go through LDS and the sequence's first 64 keys are read
// together with the accepted length and the bonus, so only the payload gather
// waits on the decision.
__global__ __launch_bounds__(WG) void k_lookup(const int32_t* keys, const int32_t* off, const int32_t* payload,
                                               int B, int K, int Bgt, const int32_t* acc, const int32_t* bonus,
                                               int32_t* hit, int32_t* slot, int32_t* toks, int64_t V,
                                               uint64_t seed, int fill) {
  __shared__ int so[MAX_K1 + 1];
  if ((int)threadIdx.x <= K + 1) so[threadIdx.x] = off[threadIdx.x];
  const int b = blockIdx.x * NWAVE + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const bool live = b < B;
  const int k = live ? acc[b] : -1, y = live ? bonus[b] : 0;
  const int key0 = (live && lane < Bgt) ? keys[(int64_t)b * Bgt + lane] : 0;
  lds_sync();
  if (!live) return;
  int found = -1;
  if (k >= 0 && k <= K) {
    const int lo = max(so[k], 0), hi = min(so[k + 1], Bgt);
    for (int s0 = lo; s0 < hi; s0 += 64) {
      const int sl = s0 + lane;
      const int sh = __shfl(key0, sl & 63);  // every lane takes part in the shuffle
      const int kv = sl < 64 ? sh : keys[(int64_t)b * Bgt + min(sl, Bgt - 1)];
      const uint64_t m = __ballot(sl < hi && kv == y);
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
    toks[(int64_t)b * K + i] = found >= 0 ? payload[((int64_t)b * Bgt + found) * K + i]
                               : fill     ? fallback_token(seed, b, i, V)
                                          : -1;
}

// Keys of every (sequence, slot): slot sl of depth k (off[k] <= sl < off[k+1])
// holds entry sl - off[k] of that depth's top list.  The depth offsets go
// through LDS.
__global__ __launch_bounds__(WG) void k_cache_keys(const int32_t* topf, int ldf, const int32_t* off, int B, int K,
                                                   int Bgt, int32_t* keys) {
  __shared__ int so[MAX_K1 + 1];
  if ((int)threadIdx.x <= K + 1) so[threadIdx.x] = off[threadIdx.x];
  lds_sync();
  const int64_t t = (int64_t)blockIdx.x * WG + threadIdx.x;
  if (t >= (int64_t)B * Bgt) return;
  const int b = (int)(t / Bgt), sl = (int)(t - (int64_t)b * Bgt);
  int kk = -1, i = 0;
  for (int k = K; k >= 0; --k)  // descending: the first depth whose range holds sl wins
    if (sl >= so[k] && sl < so[k + 1]) {
      kk = k;
      i = sl - so[k];
    }
  keys[t] = (kk >= 0 && i < ldf) ? topf[((int64_t)b * (K + 1) + kk) * ldf + i] : -1;
}

}  // namespace ssd
