// Router of the Beam MoE block on gfx950: fp32 logits on MFMA, then the
// group-limited top-k selection, one wavefront per token.
//
// Beam launch post ("Introducing Beam"), section "Mixture of Experts": all
// 256 experts are scored with a sigmoid, split into 8 groups of 32, the 4
// groups with the best sum of their two top scores are kept and the top 8
// experts inside them are chosen; their weights are normalised. Section
// "Residual Stream": the router runs in fp32. transformers model doc "Beam",
// section "Overview": a learned per-expert bias balances load (it shifts the
// selection key only); n_group / topk_group name the group parameters.
#include "common.h"
#include "internal.h"

namespace beam {

// z[t, e] = sum_h x[t, h] * W[e, h] in fp32.
//
// The workgroup (4 waves) owns a tile of 16*MW tokens x 16*NB experts; the
// waves split either the tokens (MW) or the reduction (KS), MW * KS = 4.
// Each wave walks its K range 16 values at a time with 16x16x4 fp32 MFMAs.
// A lane loads four consecutive k values of one row; MFMA j of the step
// consumes element j of every lane, so the four MFMAs together cover the 16
// k values. Each j keeps its own accumulator (shorter rounding chains); the
// four are summed in a fixed order, and K splits are summed through LDS in
// wave order, so the result does not depend on scheduling.
template <typename XT, int MW, int KS, int NB>
__global__ __launch_bounds__(256) void router_logits_kernel(const XT* __restrict__ x,
                                                            const float* __restrict__ W,
                                                            float* __restrict__ z, int T, int H) {
  static_assert(MW * KS == 4, "four waves");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave % MW, ks = wave / MW;
  const int r = lane & 15, g = lane >> 4;
  const int tok0 = blockIdx.x * (16 * MW) + wm * 16;
  const int e0 = blockIdx.y * (16 * NB);
  const int kper = H / KS;
  const int kb = ks * kper;

  const int tok = min(tok0 + r, T - 1);
  const XT* xrow = x + (size_t)tok * H + kb + 4 * g;
  const float* wrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) wrow[nb] = W + (size_t)(e0 + nb * 16 + r) * H + kb + 4 * g;

  f32x4 acc[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[nb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k = 0; k < kper; k += 16) {
    float a[4];
    if constexpr (sizeof(XT) == 4) {
      u32x4 v = ld16(xrow + k);
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = __uint_as_float(v[j]);
    } else {
      u32x2 v = *reinterpret_cast<const u32x2*>(xrow + k);
      a[0] = bf16_bits_to_f32(v[0] & 0xffffu);
      a[1] = bf16_bits_to_f32(v[0] >> 16);
      a[2] = bf16_bits_to_f32(v[1] & 0xffffu);
      a[3] = bf16_bits_to_f32(v[1] >> 16);
    }
    u32x4 b[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b[nb] = ld16(wrow[nb] + k);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb][j] = mfma_f32(a[j], __uint_as_float(b[nb][j]), acc[nb][j]);
  }

  f32x4 res[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) res[nb] = (acc[nb][0] + acc[nb][1]) + (acc[nb][2] + acc[nb][3]);

  if constexpr (KS == 1) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = tok0 + 4 * g + i;
        if (row < T) z[(size_t)row * kExperts + e0 + nb * 16 + r] = res[nb][i];
      }
  } else {
    constexpr int TM = 16 * MW, TN = 16 * NB;
    __shared__ float red[KS][TM][TN];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[ks][wm * 16 + 4 * g + i][nb * 16 + r] = res[nb][i];
    __syncthreads();
    for (int q = threadIdx.x; q < TM * TN; q += 256) {
      const int rl = q / TN, cl = q % TN;
      float s = red[0][rl][cl];
#pragma unroll
      for (int kk = 1; kk < KS; ++kk) s += red[kk][rl][cl];
      const int row = blockIdx.x * TM + rl;
      if (row < T) z[(size_t)row * kExperts + e0 + cl] = s;
    }
  }
}

// Best (key, index) of two candidates: larger key, equal keys to the lower
// index; idx < 0 marks "no candidate".
__device__ __forceinline__ void take_better(float& k, int& i, float ok, int oi) {
  const bool other = (oi >= 0) && (i < 0 || ok > k || (ok == k && oi < i));
  k = other ? ok : k;
  i = other ? oi : i;
}

// One wave per token. Lane l holds experts 4l..4l+3. A group of
// 256/n_group experts spans lpg = 64/n_group lanes.
__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ z,
                                                     const float* __restrict__ bias, int T,
                                                     int n_group, int topk_group, int top_k,
                                                     int32_t* __restrict__ idx,
                                                     float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;

  const u32x4 zv = ld16(z + (size_t)t * kExperts + 4 * lane);
  const u32x4 bv = ld16(bias + 4 * lane);
  float s[4], key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[i] = sigmoid_f32(__uint_as_float(zv[i]));
    const float kk = s[i] + __uint_as_float(bv[i]);
    key[i] = (kk == kk) ? kk : -INFINITY;  // a NaN key ranks below every number
  }

  // Sum of the two largest keys of the group (values, so equal keys both count).
  float t1 = fmaxf(key[0], key[1]), t2 = fminf(key[0], key[1]);
#pragma unroll
  for (int i = 2; i < 4; ++i) {
    const float v = key[i];
    t2 = fmaxf(t2, fminf(t1, v));
    t1 = fmaxf(t1, v);
  }
  const int lpg = 64 / n_group;
  for (int off = 1; off < lpg; off <<= 1) {
    const float o1 = __shfl_xor(t1, off), o2 = __shfl_xor(t2, off);
    const float n2 = fmaxf(fminf(t1, o1), fmaxf(t2, o2));
    t1 = fmaxf(t1, o1);
    t2 = n2;
  }
  const float gscore = t1 + t2;
  const int grp = lane / lpg;

  // Rank of this lane's group; kept if fewer than topk_group groups beat it.
  int rank = 0;
  for (int gg = 0; gg < n_group; ++gg) {
    const float sc = __shfl(gscore, gg * lpg);
    rank += (sc > gscore || (sc == gscore && gg < grp)) ? 1 : 0;
  }
  uint32_t avail = (rank < topk_group) ? 0xFu : 0u;

  // top_k rounds of a wave-wide argmax over the remaining candidates.
  float sum = 0.f, my_s = 0.f;
  int my_i = 0;
  for (int j = 0; j < top_k; ++j) {
    float bk = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if ((avail >> i) & 1u) take_better(bk, bi, key[i], 4 * lane + i);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ok = __shfl_xor(bk, off);
      const int oi = __shfl_xor(bi, off);
      take_better(bk, bi, ok, oi);
    }
    // bi is the same on every lane; at least top_k candidates exist, so bi >= 0.
    const int owner = bi >> 2, slot = bi & 3;
    if (lane == owner) avail &= ~(1u << slot);
    const float sv = (slot == 0) ? s[0] : (slot == 1) ? s[1] : (slot == 2) ? s[2] : s[3];
    const float ws = __shfl(sv, owner);
    sum += ws;
    if (lane == j) {
      my_i = bi;
      my_s = ws;
    }
  }
  if (lane < top_k) {
    idx[(size_t)t * top_k + lane] = my_i;
    wout[(size_t)t * top_k + lane] = my_s / sum;
  }
}

hipError_t launch_router_logits(const void* x, int x_f32, const float* W, float* z, int T, int H,
                                hipStream_t st) {
  // Few tokens: 16x16 tiles with the reduction split over the 4 waves, so
  // the 5 MB router matrix is streamed by many workgroups. Many tokens:
  // 64x64 tiles, one wave per 16 tokens, fewer re-reads of W and x.
  if (T <= 1024) {
    dim3 grid((T + 15) / 16, kExperts / 16);
    if (x_f32)
      router_logits_kernel<float, 1, 4, 1><<<grid, 256, 0, st>>>((const float*)x, W, z, T, H);
    else
      router_logits_kernel<uint16_t, 1, 4, 1><<<grid, 256, 0, st>>>((const uint16_t*)x, W, z, T, H);
  } else {
    dim3 grid((T + 63) / 64, kExperts / 64);
    if (x_f32)
      router_logits_kernel<float, 4, 1, 4><<<grid, 256, 0, st>>>((const float*)x, W, z, T, H);
    else
      router_logits_kernel<uint16_t, 4, 1, 4><<<grid, 256, 0, st>>>((const uint16_t*)x, W, z, T, H);
  }
  return hipGetLastError();
}

hipError_t launch_select(const float* z, const float* bias, int T, int n_group, int topk_group,
                         int top_k, int32_t* idx, float* w, hipStream_t st) {
  select_kernel<<<(T + 3) / 4, 256, 0, st>>>(z, bias, T, n_group, topk_group, top_k, idx, w);
  return hipGetLastError();
}

}  // namespace beam
