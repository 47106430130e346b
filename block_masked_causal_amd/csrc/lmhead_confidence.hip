// LM-head GEMM + per-position confidence for gfx950.
//
// MARS reuses the unchanged LM head to score all B mask positions in one
// forward, and the confidence of a position is its maximum softmax
// probability max_v p(x_t = v) (gist.science explainer on "MARS: Enabling
// Autoregressive Models Multi-Token Generation", sections 2C and 3;
// papernotes.org notes, key design 3 / 关键设计 3).
//
//  * lmhead_gemm_kernel: logits[N, V] = hidden[N, D] . W[V, D]^T on the
//    32x32x16 bf16 MFMA with fp32 accumulation. A 512-thread workgroup owns
//    all of up to 256 rows and 320 vocabulary entries, so each weight row is
//    read from HBM once; K is staged 32 at a time through a 4-stage LDS ring
//    filled by direct global->LDS loads (three stages in flight). With
//    logits == NULL the epilogue reduces the tile to per-row confidence
//    partials instead of storing logits (conf_merge_wide_kernel finishes).
//  * conf_partial_kernel: a row is cut into chunks; each workgroup streams one
//    chunk once, keeping per-thread (max, first argmax, sum of exp relative to
//    the running max), and reduces them in the workgroup (sums in fp64).
//  * conf_merge_kernel: combines the chunks of a row in a fixed order:
//    top_id = lowest index attaining the maximum, p_max = 1 / sum exp(l - m).
//  * conf_row_kernel: with at least 256 rows, one 1024-thread workgroup per
//    row does both in one pass (no partials, no second launch).
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "mars_common.hpp"

using namespace mars;

namespace {

// Per-row confidence partial over a slice of the vocabulary.
struct ConfPart {
  float m;
  int32_t idx;
  double s;  // sum of exp(l - m) over the chunk
};


// Combine (m1, i1, s1) with (m2, i2, s2); ties in m keep the lower index.
__device__ __forceinline__ void conf_combine(float& m1, int& i1, double& s1, float m2, int i2,
                                             double s2) {
  const float M = fmaxf(m1, m2);
  const double w1 = m1 == -INFINITY ? 0.0 : (double)fast_exp2((m1 - M) * kLog2e);
  const double w2 = m2 == -INFINITY ? 0.0 : (double)fast_exp2((m2 - M) * kLog2e);
  const int idx = m1 > m2 ? i1 : (m2 > m1 ? i2 : min(i1, i2));
  s1 = s1 * w1 + s2 * w2;
  m1 = M;
  i1 = idx;
}


// ------------------------------------------------------------------ GEMM ----
// Workgroup tile: GM rows (all positions, up to 256) x GN vocabulary entries;
// 8 waves as 4 (rows) x 2 (vocab), each wave 64 x 160 outputs, so each seven
// fragments read from LDS feed ten MFMAs and each weight row is read from HBM
// once. GN = 320 because 152064 / 320 = 476 tiles fill two rounds of one tile
// per CU on 256 CUs (256-wide tiles left a 2.32-round grid). K advances GK = 32 per stage through a ring of GSTAGES = 4
// LDS stages filled by direct global->LDS loads: three stages are always in
// flight while one is multiplied (one 64-wide stage in flight, as a register
// staged pipeline allows, left each workgroup waiting on memory latency).
constexpr int GM = 256;
constexpr int GN = 320;
constexpr int GN_TAIL = 64;  // tail tiles: divide GN, so none straddles a packed tile
constexpr int GT = 512;                 // threads per workgroup
constexpr int GK = 32;                  // K per stage
constexpr int GSTAGES = 4;
constexpr int GCPR = GK / 8;            // 16-byte chunks per tile row
constexpr int GROWS_BLK = 64 / GCPR;    // rows per 1 KiB direct-load block
constexpr int GABLK = GM / GROWS_BLK;   // blocks per hidden tile

// Rows sit in LDS unpadded; chunk c of row r is stored at chunk c ^ gswz(r),
// which keeps 16 consecutive rows read at one chunk on 16 distinct groups of
// 4 banks (64 banks).
__device__ __forceinline__ int gswz(int r) { return (r >> 2) & 3; }

struct GemmArgs {
  const bf16_t* hidden;
  const bf16_t* w;   // [V, D] rows, or packed: [nvt][D / GK][GN][GK] (one stage contiguous)
  int packed;
  int v_base;        // first vocabulary entry of this launch's tiles
  int tile0;         // index of this launch's first tile among the row's partials
  float* logits;     // unfused: [N, V] fp32
  ConfPart* part;    // fused: [N][nvt] partials, one per vocabulary tile
  int32_t* status;
  int N, D, V, nvt;
};

// logits^T = W . hidden^T: the MFMA A operand is a 32-entry slice of the
// vocabulary, B a 32-position slice, so lane (j, hf) of tile (va, pb) holds
// position n0 + wn*64 + 32 pb + j and vocabulary entries
// v0 + wv*TN/2 + 32 va + 8 (r / 4) + 4 hf + r % 4, r = 0..15. A position's
// TN entries of the workgroup tile are thus TN/4 values in each of 4 lanes
// (two halves of two waves): FUSED reduces them in registers to the
// confidence partial (max, first argmax, sum exp(l - max)) and writes no
// logits.
// TN: vocabulary entries per workgroup (GN, or GN_TAIL for the tail tiles).
// A stage is GM / 16 + TN / 16 direct loads of 1 KiB; when they do not split
// evenly over the 8 waves, the first GXTRA waves issue one more, and each wave
// waits for its own count.
template <bool FUSED, int TN>
__global__ __launch_bounds__(GT, 2) void lmhead_gemm_kernel(GemmArgs p) {
  constexpr int WNT = TN / 64;            // 32-wide vocab MFMA tiles per wave
  constexpr int GWBLK = TN / GROWS_BLK;   // blocks per weight tile
  constexpr int GNBLK = GABLK + GWBLK;                // 1 KiB blocks per stage
  constexpr int GBPW = (GNBLK + GT / 64 - 1) / (GT / 64);  // blocks of the busiest wave
  constexpr int GXTRA = GNBLK % (GT / 64);  // waves below this issue GBPW, the rest GBPW - 1
  constexpr int GSTAGE_EL = (GM + TN) * GK;          // elements per stage
  static_assert(TN % 64 == 0 && 2 * GBPW < 16, "stage split");
  __shared__ __attribute__((aligned(16))) bf16_t st0[GSTAGE_EL];
  __shared__ __attribute__((aligned(16))) bf16_t st1[GSTAGE_EL];
  __shared__ __attribute__((aligned(16))) bf16_t st2[GSTAGE_EL];
  __shared__ __attribute__((aligned(16))) bf16_t st3[GSTAGE_EL];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, hf = lane >> 5;
  const int wn = w >> 1, wv = w & 1;
  const int v0 = p.v_base + blockIdx.x * TN;
  const int n0 = blockIdx.y * GM;
  const int nk = p.D / GK;

  // buffer views of this tile's rows: rows past N (or V) read as zeros
  const u32x4 rh = rsrc_words(p.hidden + (size_t)n0 * p.D,
                              (uint32_t)((size_t)min(GM, p.N - n0) * p.D * sizeof(bf16_t)));
  // the packed layout holds every GN-row tile whole (rows past V are zeros);
  // a narrower tile reads its rows inside one packed tile
  const int prow0 = v0 % GN;  // first row inside the packed tile
  const u32x4 rw =
      p.packed ? rsrc_words(p.w + (size_t)(v0 / GN) * GN * p.D,
                            (uint32_t)((size_t)GN * p.D * sizeof(bf16_t)))
               : rsrc_words(p.w + (size_t)v0 * p.D,
                            (uint32_t)((size_t)min(TN, p.V - v0) * p.D * sizeof(bf16_t)));
  // stage kt: wave w fills blocks w, w + 8, ... (hidden tile first, then weights)
  auto issue = [&](int kt, bf16_t* st) {
#pragma unroll
    for (int i = 0; i < GBPW; ++i) {
      const int blk = w + (GT / 64) * i;
      if (blk >= GNBLK) break;  // wave-uniform
      const bool is_a = blk < GABLK;
      const int rb = (is_a ? blk : blk - GABLK) * GROWS_BLK;
      const int row = rb + lane / GCPR, slot = lane % GCPR;
      // row-major: 64 bytes of each of the tile's rows; packed: one
      // contiguous 16 KiB block per stage
      const uint32_t off =
          (is_a || !p.packed)
              ? (uint32_t)((size_t)row * p.D * sizeof(bf16_t)) +
                    (uint32_t)(kt * GK * sizeof(bf16_t)) + 16 * (slot ^ gswz(row))
              : (uint32_t)(kt * GN * GK * sizeof(bf16_t)) +
                    (uint32_t)((prow0 + row) * GK * sizeof(bf16_t)) + 16 * (slot ^ gswz(row));
      lds_dma16(is_a ? rh : rw, st + (is_a ? 0 : GM * GK) + rb * GK, off);
    }
  };

  f32x16 acc[WNT][2];
#pragma unroll
  for (int a = 0; a < WNT; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  // fragment offsets: row base + 32 t + j has the swizzle of j; chunk 2 ks + hf
  const int sw = gswz(j);
  int koff[GK / 16];
#pragma unroll
  for (int ks = 0; ks < GK / 16; ++ks) koff[ks] = 8 * ((2 * ks + hf) ^ sw);
  auto compute = [&](const bf16_t* st) {
    const bf16_t* A = st;
    const bf16_t* Wt = st + GM * GK;
#pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks) {
      bf16x8 wf[WNT], hfr[2];
#pragma unroll
      for (int t = 0; t < WNT; ++t)
        wf[t] = *(const bf16x8*)(Wt + (wv * (TN / 2) + 32 * t + j) * GK + koff[ks]);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        hfr[t] = *(const bf16x8*)(A + (wn * 64 + 32 * t + j) * GK + koff[ks]);
#pragma unroll
      for (int a = 0; a < WNT; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma32(wf[a], hfr[b], acc[a][b]);
    }
  };

  // wait until at most S stages of this wave's loads are in flight (a wave's
  // loads per stage: GBPW, or GBPW - 1 past the first GXTRA waves)
  auto wait_stages = [&](auto s_tag) {
    constexpr int S = decltype(s_tag)::value;
    if (GXTRA == 0 || w < GXTRA)
      wait_vm_upto<S * GBPW>();
    else
      wait_vm_upto<S * (GBPW - 1)>();
  };
  // prologue: stages 0..2 in flight, wait for stage 0
  issue(0, st0);
  if (nk > 1) issue(1, st1);
  if (nk > 2) issue(2, st2);
  if (nk > 2)
    wait_stages(std::integral_constant<int, 2>{});
  else if (nk > 1)
    wait_stages(std::integral_constant<int, 1>{});
  else
    wait_vm_upto<0>();
  __builtin_amdgcn_s_barrier();

  // step kt reads stage kt % 4 and refills the stage step kt - 1 read
  auto step = [&](int kt, auto s_tag) {
    constexpr int S = decltype(s_tag)::value;
    bf16_t* const cur = S == 0 ? st0 : S == 1 ? st1 : S == 2 ? st2 : st3;
    bf16_t* const ref = S == 0 ? st3 : S == 1 ? st0 : S == 2 ? st1 : st2;
    if (kt + 3 < nk) issue(kt + 3, ref);
    compute(cur);
    // stage kt + 1 has landed once at most the stages issued after it are in flight
    if (kt + 3 < nk)
      wait_stages(std::integral_constant<int, 2>{});
    else if (kt + 2 < nk)
      wait_stages(std::integral_constant<int, 1>{});
    else
      wait_vm_upto<0>();
    __builtin_amdgcn_s_barrier();
  };
  for (int kt = 0; kt < nk; kt += GSTAGES) {
    step(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1>{});
    if (kt + 2 < nk) step(kt + 2, std::integral_constant<int, 2>{});
    if (kt + 3 < nk) step(kt + 3, std::integral_constant<int, 3>{});
  }
  bf16_t* const gl = st0;  // free after the K loop: the epilogue's exchange area

  const int vb = v0 + wv * (TN / 2) + 4 * hf;  // + 32 va + 8 (r / 4) + r % 4
  if constexpr (!FUSED) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int n = n0 + wn * 64 + 32 * b + j;
      if (n >= p.N) continue;
      float* row = p.logits + (size_t)n * p.V;
#pragma unroll
      for (int a = 0; a < WNT; ++a)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int v = vb + 32 * a + 8 * g;  // 4 consecutive entries; V % 4 == 0
          if (v < p.V)
            *(f32x4*)(row + v) = f32x4{acc[a][b][4 * g], acc[a][b][4 * g + 1],
                                       acc[a][b][4 * g + 2], acc[a][b][4 * g + 3]};
        }
    }
  } else {
    // exchange area for the two waves sharing a position (the K loop is done)
    float* xm = (float*)gl;
    int* xi = (int*)(xm + 4 * 64);
    double* xs = (double*)(xi + 4 * 64);
    bool bad = false;
    float pm[2];
    int pi[2];
    double ps[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float m = -INFINITY;
#pragma unroll
      for (int a = 0; a < WNT; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int v = vb + 32 * a + 8 * (r >> 2) + (r & 3);
          if (v < p.V) m = fmaxf(m, acc[a][b][r]);
        }
      // the lowest entry equal to the max: walk the lane's entries downwards
      int idx = 0x7FFFFFFF;
      float sum = 0.f;
#pragma unroll
      for (int a = WNT - 1; a >= 0; --a)
#pragma unroll
        for (int r = 15; r >= 0; --r) {
          const int v = vb + 32 * a + 8 * (r >> 2) + (r & 3);
          const float x = acc[a][b][r];
          if (v < p.V) {
            idx = x == m ? v : idx;
            sum += fast_exp2((x - m) * kLog2e);
          }
        }
      if (m == -INFINITY) sum = 0.f;  // no entry of this lane lies below V
      bad |= (m != -INFINITY) && !(isfinite(m) && isfinite(sum));
      double sd = (double)sum;
      // the other half of the wave holds the interleaved entries of the same position
      const auto sm_ = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m),
                                                        false, false);
      const auto si_ = __builtin_amdgcn_permlane32_swap((uint32_t)idx, (uint32_t)idx, false,
                                                        false);
      const uint64_t sb = __builtin_bit_cast(uint64_t, sd);
      const auto slo = __builtin_amdgcn_permlane32_swap((uint32_t)sb, (uint32_t)sb, false,
                                                        false);
      const auto shi = __builtin_amdgcn_permlane32_swap((uint32_t)(sb >> 32),
                                                        (uint32_t)(sb >> 32), false, false);
      // the swap leaves the lower half's values in one result and the upper
      // half's in the other, in every lane; the combination is symmetric
      // (commutative sum, ties to the lower index), so their order is immaterial
      m = __uint_as_float(sm_[0]);
      idx = (int)si_[0];
      sd = __builtin_bit_cast(double, ((uint64_t)shi[0] << 32) | (uint64_t)slo[0]);
      conf_combine(m, idx, sd, __uint_as_float(sm_[1]), (int)si_[1],
                   __builtin_bit_cast(double, ((uint64_t)shi[1] << 32) | (uint64_t)slo[1]));
      pm[b] = m;
      pi[b] = idx;
      ps[b] = sd;
    }
    if (bad) status_or(p.status, MARS_STATUS_NONFINITE);
    if (wv == 1 && hf == 0) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int slot = wn * 64 + 32 * b + j;
        xm[slot] = pm[b];
        xi[slot] = pi[b];
        xs[slot] = ps[b];
      }
    }
    __syncthreads();
    if (wv == 0 && hf == 0) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int slot = wn * 64 + 32 * b + j;
        const int n = n0 + slot;
        conf_combine(pm[b], pi[b], ps[b], xm[slot], xi[slot], xs[slot]);
        if (n < p.N) {
          ConfPart out;
          out.m = pm[b];
          out.idx = pi[b];
          out.s = ps[b];
          p.part[(size_t)n * p.nvt + p.tile0 + blockIdx.x] = out;
        }
      }
    }
  }
}

// ------------------------------------------------------------ confidence ----
struct ConfArgs {
  const float* logits;
  int32_t* top_id;
  float* p_max;
  ConfPart* part;
  int32_t* status;
  int N, V, nchunk, chunk;  // chunk: elements per chunk, multiple of 4
};

__global__ __launch_bounds__(256) void conf_partial_kernel(ConfArgs p) {
  const int c = blockIdx.x, row = blockIdx.y;
  const int tid = threadIdx.x;
  const int lo = c * p.chunk;
  const int hi = min(p.V, lo + p.chunk);
  const float* L = p.logits + (size_t)row * p.V;

  float m = -INFINITY;
  int idx = 0x7FFFFFFF;
  float s = 0.f;
  bool bad = false;
  for (int i = lo + 4 * tid; i < hi; i += 4 * 256) {
    const f32x4 x = *(const f32x4*)(L + i);
    bad |= !(isfinite(x[0]) && isfinite(x[1]) && isfinite(x[2]) && isfinite(x[3]));
    const float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (bm > m) {
      s = m == -INFINITY ? 0.f : s * fast_exp2((m - bm) * kLog2e);
      m = bm;
      idx = x[0] == bm ? i : (x[1] == bm ? i + 1 : (x[2] == bm ? i + 2 : i + 3));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) s += fast_exp2((x[e] - m) * kLog2e);
  }
  if (bad) status_or(p.status, MARS_STATUS_NONFINITE);

  double sd = (double)s;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o);
    const int i2 = __shfl_xor(idx, o);
    const double s2 = __shfl_xor(sd, o);
    conf_combine(m, idx, sd, m2, i2, s2);
  }
  __shared__ float sm[4];
  __shared__ int si[4];
  __shared__ double ss[4];
  const int wv = tid >> 6;
  if ((tid & 63) == 0) {
    sm[wv] = m;
    si[wv] = idx;
    ss[wv] = sd;
  }
  __syncthreads();
  if (tid == 0) {
    float M = sm[0];
    int I = si[0];
    double S = ss[0];
    for (int k = 1; k < 4; ++k) conf_combine(M, I, S, sm[k], si[k], ss[k]);
    ConfPart out;
    out.m = M;
    out.idx = I;
    out.s = S;
    p.part[(size_t)row * p.nchunk + c] = out;
  }
}

// Confidence of whole rows, one 1024-thread workgroup per row (used when
// there are enough rows to fill the GPU, N >= kRowKernelMinRows): no partials
// and no merge launch. Each thread keeps four 16-byte loads in flight and folds
// its elements in index order; then a fixed butterfly over each wave and a
// fixed order over the 16 waves, sums in fp64.
constexpr int kRowThreads = 1024;
constexpr int kRowKernelMinRows = 256;
__global__ __launch_bounds__(kRowThreads) void conf_row_kernel(ConfArgs p) {
  constexpr int U = 4;  // loads in flight per thread
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const float* L = p.logits + (size_t)row * p.V;
  float m = -INFINITY;
  int idx = 0x7FFFFFFF;
  float s = 0.f;
  bool bad = false;
  auto fold = [&](const f32x4& x, int i) {
    bad |= !(isfinite(x[0]) && isfinite(x[1]) && isfinite(x[2]) && isfinite(x[3]));
    const float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (bm > m) {
      s = m == -INFINITY ? 0.f : s * fast_exp2((m - bm) * kLog2e);
      m = bm;
      idx = x[0] == bm ? i : (x[1] == bm ? i + 1 : (x[2] == bm ? i + 2 : i + 3));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) s += fast_exp2((x[e] - m) * kLog2e);
  };
  constexpr int step = 4 * kRowThreads;
  int i = 4 * tid;
  for (; i + (U - 1) * step < p.V; i += U * step) {
    f32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = *(const f32x4*)(L + i + u * step);
#pragma unroll
    for (int u = 0; u < U; ++u) fold(x[u], i + u * step);
  }
  for (; i < p.V; i += step) fold(*(const f32x4*)(L + i), i);
  if (bad) status_or(p.status, MARS_STATUS_NONFINITE);

  double sd = (double)s;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o);
    const int i2 = __shfl_xor(idx, o);
    const double s2 = __shfl_xor(sd, o);
    conf_combine(m, idx, sd, m2, i2, s2);
  }
  constexpr int NWV = kRowThreads / 64;
  __shared__ float sm[NWV];
  __shared__ int si[NWV];
  __shared__ double ss[NWV];
  const int wv = tid >> 6;
  if ((tid & 63) == 0) {
    sm[wv] = m;
    si[wv] = idx;
    ss[wv] = sd;
  }
  __syncthreads();
  if (tid == 0) {
    float M = sm[0];
    int I = si[0];
    double S = ss[0];
    for (int k = 1; k < NWV; ++k) conf_combine(M, I, S, sm[k], si[k], ss[k]);
    p.top_id[row] = I == 0x7FFFFFFF ? 0 : I;
    p.p_max[row] = (float)(1.0 / S);
  }
}

__global__ __launch_bounds__(256) void conf_merge_kernel(ConfArgs p) {
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row >= p.N) return;
  const ConfPart* pr = p.part + (size_t)row * p.nchunk;
  float M = pr[0].m;
  int I = pr[0].idx;
  double S = pr[0].s;
  for (int c = 1; c < p.nchunk; ++c) conf_combine(M, I, S, pr[c].m, pr[c].idx, pr[c].s);
  p.top_id[row] = I == 0x7FFFFFFF ? 0 : I;
  p.p_max[row] = (float)(1.0 / S);
}

// Merge of many partials per row (the fused path: one per vocabulary tile): one workgroup per row, each thread folds a strided subset in order,
// then a fixed butterfly over the wave and a fixed order over the 4 waves.
__global__ __launch_bounds__(256) void conf_merge_wide_kernel(ConfArgs p) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const ConfPart* pr = p.part + (size_t)row * p.nchunk;
  float m = -INFINITY;
  int idx = 0x7FFFFFFF;
  double s = 0.0;
  for (int c = tid; c < p.nchunk; c += 256) conf_combine(m, idx, s, pr[c].m, pr[c].idx, pr[c].s);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o);
    const int i2 = __shfl_xor(idx, o);
    const double s2 = __shfl_xor(s, o);
    conf_combine(m, idx, s, m2, i2, s2);
  }
  __shared__ float sm[4];
  __shared__ int si[4];
  __shared__ double ss[4];
  const int wv = tid >> 6;
  if ((tid & 63) == 0) {
    sm[wv] = m;
    si[wv] = idx;
    ss[wv] = s;
  }
  __syncthreads();
  if (tid == 0) {
    for (int k = 1; k < 4; ++k) conf_combine(sm[0], si[0], ss[0], sm[k], si[k], ss[k]);
    p.top_id[row] = si[0] == 0x7FFFFFFF ? 0 : si[0];
    p.p_max[row] = (float)(1.0 / ss[0]);
  }
}

// Weight packing: W [V, D] -> [nvt][D / GK][GN][GK], rows past V zero, so that
// every GEMM stage reads one contiguous 20 KiB block of weights (a row-major
// stage is 64 bytes from each of 320 rows 2D bytes apart). One 16-byte chunk
// per thread, in packed order.
__global__ __launch_bounds__(256) void lmhead_pack_kernel(const bf16_t* __restrict__ w,
                                                          bf16_t* __restrict__ wp, int D,
                                                          int V, long long chunks) {
  constexpr int CPR = GK / 8;  // chunks per packed row
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < chunks;
       i += (long long)gridDim.x * 256) {
    const long long tile = i / (GN * CPR);
    const int within = (int)(i % (GN * CPR));
    const int r = within / CPR, c8 = within % CPR;
    const long long vt = tile / (D / GK);
    const int kt = (int)(tile % (D / GK));
    const long long v = vt * GN + r;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (v < V) val = *(const u32x4*)(w + v * D + kt * GK + c8 * 8);
    *(u32x4*)(wp + i * 8) = val;
  }
}

void conf_layout(int N, int V, int* nchunk, int* chunk) {
  int c = std::max(1, std::min(32, (2048 + N - 1) / N));
  c = std::min(c, std::max(1, (V + 1023) / 1024));
  int ch = (V + c - 1) / c;
  ch = (ch + 3) & ~3;
  c = (V + ch - 1) / ch;
  *nchunk = c;
  *chunk = ch;
}

}  // namespace

namespace {
// One GN-wide tile per workgroup and one workgroup per CU at a time (the LDS
// ring): tiles run in rounds of one per CU. When the last round's tiles, cut
// into GN_TAIL-wide tiles, would still fit one round, they run that way and
// finish well before a full round (the vocabulary order of the partials is
// kept: main tiles first, then the tail's).
// The GEMM's vocabulary tiling: main_tiles of GN entries, then tail_tiles of
// GN_TAIL. Their sum is the number of confidence partials per row.
void gemm_tiles(int V, int row_tiles, int* main_tiles, int* tail_tiles) {
  const int full = (V + GN - 1) / GN;
  const int ncu = mars_cu_count();
  int m = full;
  if (row_tiles == 1 && ncu > 0 && full > ncu) {
    const int r = full % ncu;
    if (r > 0 && (GN / GN_TAIL) * r <= ncu) m = full - r;
  }
  const int tail_v = V - m * GN;  // entries left to the narrow tiles
  *main_tiles = m;
  *tail_tiles = tail_v > 0 ? (tail_v + GN_TAIL - 1) / GN_TAIL : 0;
}

template <bool FUSED>
int launch_gemm(GemmArgs g, int row_tiles, hipStream_t st) {
  int main_tiles, tail_tiles;
  gemm_tiles(g.V, row_tiles, &main_tiles, &tail_tiles);
  g.nvt = main_tiles + tail_tiles;
  g.v_base = 0;
  g.tile0 = 0;
  if (main_tiles > 0)
    hipLaunchKernelGGL((lmhead_gemm_kernel<FUSED, GN>), dim3(main_tiles, row_tiles), dim3(GT),
                       0, st, g);
  if (tail_tiles > 0) {
    g.v_base = main_tiles * GN;
    g.tile0 = main_tiles;
    hipLaunchKernelGGL((lmhead_gemm_kernel<FUSED, GN_TAIL>), dim3(tail_tiles, row_tiles),
                       dim3(GT), 0, st, g);
  }
  return g.nvt;
}
}  // namespace

extern "C" size_t mars_lmhead_workspace_bytes(int32_t N, int32_t V) {
  if (N < 1 || V < 4 || V % 4) return 0;
  int nchunk, chunk;
  conf_layout(N, V, &nchunk, &chunk);
  // fused path: one partial per vocabulary tile; bounded by tiles of GN_TAIL
  const int nvt = (GN / GN_TAIL) * ((V + GN - 1) / GN);
  return (size_t)N * std::max(nchunk, nvt) * sizeof(ConfPart);
}

namespace {
// Argument checks shared by every LM-head entry point (not the workspace).
int check_lmhead(const void* hidden, const void* w_lm, const float* logits, int32_t N, int32_t D,
                 int32_t V, const int32_t* top_id, const float* p_max) {
  MARS_REQUIRE(top_id && p_max, MARS_ERR_NULL);
  MARS_REQUIRE(!hidden || w_lm, MARS_ERR_NULL);
  MARS_REQUIRE(hidden || logits, MARS_ERR_NULL);  // logits may be omitted only when fused
  MARS_REQUIRE(N >= 1 && V >= 4 && V % 4 == 0, MARS_ERR_SHAPE);
  MARS_REQUIRE(N <= 65535, MARS_ERR_SHAPE);  // confidence grid: one row per gridDim.y
  MARS_REQUIRE((double)N * V < 9.0e18, MARS_ERR_SHAPE);
  if (hidden) {
    MARS_REQUIRE(D >= 32 && D % 32 == 0, MARS_ERR_SHAPE);
    // buffer views address one GN-row tile with 32-bit byte offsets
    MARS_REQUIRE((double)GN * D * 2 < 4294967295.0, MARS_ERR_SHAPE);
  }
  MARS_REQUIRE(mars_aligned16(hidden) && mars_aligned16(w_lm) && mars_aligned16(logits) &&
                   mars_aligned16(top_id) && mars_aligned16(p_max),
               MARS_ERR_ALIGN);
  return MARS_OK;
}

// Bytes of partials the call actually uses: one per (row, vocabulary tile) on
// the fused path, one per (row, chunk) when the confidence reads logits.
size_t lmhead_need_bytes(bool fused, int32_t N, int32_t V) {
  int nparts;
  if (fused) {
    int main_tiles, tail_tiles;
    gemm_tiles(V, (N + GM - 1) / GM, &main_tiles, &tail_tiles);
    nparts = main_tiles + tail_tiles;
  } else {
    int chunk;
    conf_layout(N, V, &nparts, &chunk);
  }
  return (size_t)N * nparts * sizeof(ConfPart);
}

// Enqueues the call with `part` (16-byte aligned, large enough) as the partials.
int launch_lmhead(const void* hidden, const void* w_lm, int packed, float* logits, int32_t N,
                  int32_t D, int32_t V, int32_t* top_id, float* p_max, ConfPart* part,
                  int32_t* status, hipStream_t st) {
  ConfArgs c;
  c.logits = logits;
  c.top_id = top_id;
  c.p_max = p_max;
  c.part = part;
  c.status = status;
  c.N = N;
  c.V = V;
  if (hidden) {
    GemmArgs g;
    g.hidden = (const bf16_t*)hidden;
    g.w = (const bf16_t*)w_lm;
    g.packed = packed;
    g.logits = logits;
    g.part = part;
    g.status = status;
    g.N = N;
    g.D = D;
    g.V = V;
    const int row_tiles = (N + GM - 1) / GM;
    const bool fused = logits == nullptr;
    const int nvt = fused ? launch_gemm<true>(g, row_tiles, st)
                          : launch_gemm<false>(g, row_tiles, st);
    if (fused) {
      c.nchunk = nvt;
      c.chunk = GN;
      hipLaunchKernelGGL(conf_merge_wide_kernel, dim3(N), dim3(256), 0, st, c);
      return mars_launch_status();
    }
  }
  conf_layout(N, V, &c.nchunk, &c.chunk);
  if (N >= kRowKernelMinRows) {
    hipLaunchKernelGGL(conf_row_kernel, dim3(N), dim3(kRowThreads), 0, st, c);
    return mars_launch_status();
  }
  hipLaunchKernelGGL(conf_partial_kernel, dim3(c.nchunk, N), dim3(256), 0, st, c);
  hipLaunchKernelGGL(conf_merge_kernel, dim3((N + 255) / 256), dim3(256), 0, st, c);
  return mars_launch_status();
}

int run_lmhead(const void* hidden, const void* w_lm, int packed, float* logits, int32_t N,
               int32_t D, int32_t V, int32_t* top_id, float* p_max, void* workspace,
               size_t workspace_bytes, int32_t* status, void* stream) {
  const int err = check_lmhead(hidden, w_lm, logits, N, D, V, top_id, p_max);
  if (err != MARS_OK) return err;
  MARS_REQUIRE(mars_aligned16(workspace), MARS_ERR_ALIGN);
  const size_t need = mars_lmhead_workspace_bytes(N, V);
  MARS_REQUIRE(workspace && workspace_bytes >= need, MARS_ERR_WORKSPACE);
  return launch_lmhead(hidden, w_lm, packed, logits, N, D, V, top_id, p_max,
                       (ConfPart*)workspace, status, (hipStream_t)stream);
}
}  // namespace

extern "C" int mars_lmhead_confidence(const void* hidden, const void* w_lm, float* logits,
                                      int32_t N, int32_t D, int32_t V, int32_t* top_id,
                                      float* p_max, void* workspace, size_t workspace_bytes,
                                      int32_t* status, void* stream) {
  return run_lmhead(hidden, w_lm, 0, logits, N, D, V, top_id, p_max, workspace,
                    workspace_bytes, status, stream);
}

// ---- the same call without a workspace argument -----------------------------
// The confidence partials live in `scratch`, a library-owned device array. In
// host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[MARS_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch`, or NULL on a HIP error.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" int mars_lmhead_confidence_noalloc(const void* hidden, const void* w_lm,
                                              float* logits, int32_t N, int32_t D, int32_t V,
                                              int32_t* top_id, float* p_max, int32_t* status,
                                              void* stream) {
  const int err = check_lmhead(hidden, w_lm, logits, N, D, V, top_id, p_max);
  if (err != MARS_OK) return err;
  const bool fused = hidden != nullptr && logits == nullptr;
  MARS_REQUIRE(lmhead_need_bytes(fused, N, V) <= (size_t)MARS_NOALLOC_SCRATCH_BYTES,
               MARS_ERR_WORKSPACE);
  void* part = scratch_address();
  MARS_REQUIRE(part != nullptr, MARS_ERR_LAUNCH);
  return launch_lmhead(hidden, w_lm, 0, logits, N, D, V, top_id, p_max, (ConfPart*)part,
                       status, (hipStream_t)stream);
}

extern "C" size_t mars_lmhead_packed_bytes(int32_t D, int32_t V) {
  if (D < 32 || D % 32 || V < 4 || V % 4) return 0;
  return (size_t)((V + GN - 1) / GN) * GN * D * sizeof(bf16_t);
}

extern "C" int mars_lmhead_pack(const void* w_lm, void* w_packed, int32_t D, int32_t V,
                                void* stream) {
  MARS_REQUIRE(w_lm && w_packed, MARS_ERR_NULL);
  MARS_REQUIRE(mars_lmhead_packed_bytes(D, V) > 0, MARS_ERR_SHAPE);
  MARS_REQUIRE((double)GN * D * 2 < 4294967295.0, MARS_ERR_SHAPE);
  MARS_REQUIRE(mars_aligned16(w_lm) && mars_aligned16(w_packed), MARS_ERR_ALIGN);
  const long long chunks = (long long)((V + GN - 1) / GN) * GN * D / 8;
  const long long blocks = std::min<long long>((chunks + 255) / 256, 1 << 20);
  hipLaunchKernelGGL(lmhead_pack_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, (const bf16_t*)w_lm, (bf16_t*)w_packed, D, V, chunks);
  return mars_launch_status();
}

extern "C" int mars_lmhead_confidence_packed(const void* hidden, const void* w_packed,
                                             float* logits, int32_t N, int32_t D, int32_t V,
                                             int32_t* top_id, float* p_max, void* workspace,
                                             size_t workspace_bytes, int32_t* status,
                                             void* stream) {
  MARS_REQUIRE(hidden && w_packed, MARS_ERR_NULL);
  return run_lmhead(hidden, w_packed, 1, logits, N, D, V, top_id, p_max, workspace,
                    workspace_bytes, status, stream);
}
