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

#include <type_traits>

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
// wave order, so the result does not depend on scheduling. With gridDim.z
// = Z > 1 the reduction is also split over Z workgroups: workgroup z covers
// the z-th of Z equal K ranges and writes its partial logits to
// z + z * T * 256 (summed in z order by the selection).
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
  const int kper = H / (KS * (int)gridDim.z);
  const int kb = ((int)blockIdx.z * KS + ks) * kper;
  z += (size_t)blockIdx.z * T * kExperts;

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

  // One 16-k step: four k values of x per lane and of each of the NB weight rows.
  auto load = [&](int k, float (&a)[4], u32x4 (&b)[NB]) {
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
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b[nb] = ld16(wrow[nb] + k);
  };
  auto step = [&](const float (&a)[4], const u32x4 (&b)[NB]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb][j] = mfma_f32(a[j], __uint_as_float(b[nb][j]), acc[nb][j]);
  };
  // U steps at a time, all their loads issued before their MFMAs, so that
  // a short K range is not a chain of one load round trip per step; the
  // order of the steps (and of the sums) is unchanged
  constexpr int U = NB == 1 ? 8 : 2;
  int k = 0;
  for (; k + 16 * U <= kper; k += 16 * U) {
    float a[U][4];
    u32x4 b[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) load(k + 16 * u, a[u], b[u]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) step(a[u], b[u]);
  }
  for (; k < kper; k += 16) {
    float a[4];
    u32x4 b[NB];
    load(k, a, b);
    step(a, b);
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

// ------------------------------------------------------------------ bf16 x 3
// With bf16 tokens the fp32 logits can run on the bf16 matrix cores without
// changing the arithmetic: every fp32 weight is the exact sum of three bf16
// values (hi = w with the low 16 bits cleared, mid = the same for w - hi,
// lo = w - hi - mid, which has at most 8 significant bits), and a bf16 x bf16
// product is exact in fp32. So x . w = x . hi + x . mid + x . lo with exact
// products and fp32 accumulation, like an fp32 dot product, at the bf16 rate.

// W [256, H] fp32 -> three bf16 matrices (hi, mid, lo), each [256, H] in the
// packed MFMA fragment order: the 16 rows x 32 columns of one operand are one
// 1 KB block, lane l = (row % 16) + 16 * (column % 32 / 8) holding 8
// consecutive columns. One thread per 8 consecutive columns of a row.
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ W, int H,
                                                           uint16_t* __restrict__ ws) {
  const int chunks = H / 8;
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q >= kExperts * chunks) return;
  const int r = q / chunks, c0 = (q - r * chunks) * 8;
  const u32x4 v0 = ld16(W + (size_t)r * H + c0), v1 = ld16(W + (size_t)r * H + c0 + 4);
  uint32_t part[3][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t u = (i < 4) ? v0[i] : v1[i - 4];
    const uint32_t hi = u & 0xffff0000u;
    const float r1 = __uint_as_float(u) - __uint_as_float(hi);  // exact
    const uint32_t mid = __float_as_uint(r1) & 0xffff0000u;
    const float lo = r1 - __uint_as_float(mid);                  // exact, <= 8 bits
    const uint32_t b[3] = {hi >> 16, mid >> 16, __float_as_uint(lo) >> 16};
#pragma unroll
    for (int sp = 0; sp < 3; ++sp) {
      if (i & 1)
        part[sp][i >> 1] |= b[sp] << 16;
      else
        part[sp][i >> 1] = b[sp];
    }
  }
  const size_t off = ((size_t)(r >> 4) * (H / 32) + (c0 >> 5)) * 512 +
                     (size_t)((r & 15) + 16 * ((c0 & 31) >> 3)) * 8;
#pragma unroll
  for (int sp = 0; sp < 3; ++sp)
    st16(ws + (size_t)sp * kExperts * H + off,
         u32x4{part[sp][0], part[sp][1], part[sp][2], part[sp][3]});
}

// Partial logits zp[kz, t, e] = sum over the kz-th K range of x[t, h] * W[e, h]
// (gridDim.z ranges), on 16x16x32 bf16 MFMAs with the split weights.
// Workgroup: 256 tokens x 128 experts, 8 waves as 4 (tokens) x 2 (experts),
// each 64 x 64. Operands go global -> LDS by DMA through a ring of 3 stages of
// 32 k: x rows (64 bytes per row, 16-byte chunk g of row r stored at position
// g ^ ((r >> 1) & 3)) and 24 weight blocks (3 parts x 8 row blocks of 1 KB).
// The weight fragment is the MFMA's first operand, so a lane ends with 4
// consecutive experts of one token, stored as one 16-byte write.
constexpr int kRxBM = 256, kRxBN = 128, kRxNS = 3;

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void router_x3_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ ws,
                      float* __restrict__ zp, int T, int H) {
  constexpr int NS = kRxNS, A_BYTES = kRxBM * 64, B_BYTES = 24 * 1024, STAGE = A_BYTES + B_BYTES;
  constexpr int PER_STAGE = 5;  // DMAs per wave per stage: 2 x rows + 3 weight blocks
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1, r = lane & 15, g = lane >> 4;
  const int tok0 = blockIdx.x * kRxBM, e0 = blockIdx.y * kRxBN;
  const int nk = (H / 32) / gridDim.z, kt0 = blockIdx.z * nk;

  const uint16_t* asrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = (wave * 2 + i) * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 1) & 3);
    asrc[i] = x + (size_t)min(tok0 + row, T - 1) * H + (size_t)kt0 * 32 + chunk * 8;
  }
  const uint16_t* bsrc[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int j = wave * 3 + i, sp = j >> 3, rb = j & 7;
    bsrc[i] = ws + (size_t)sp * kExperts * H +
              ((size_t)((e0 >> 4) + rb) * (H / 32) + kt0) * 512 + lane * 8;
  }
  auto issue = [&](int kt) {
    uint8_t* st = smem + (kt % NS) * STAGE;
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(asrc[i] + (size_t)kt * 32, st + (wave * 2 + i) * 1024);
#pragma unroll
    for (int i = 0; i < 3; ++i) dma16(bsrc[i] + (size_t)kt * 512, st + A_BYTES + (wave * 3 + i) * 1024);
  };

  int aoff[4], boff[3][4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int row = wm * 64 + f * 16 + r;
    aoff[f] = row * 64 + ((g ^ ((row >> 1) & 3)) << 4);
#pragma unroll
    for (int sp = 0; sp < 3; ++sp) boff[sp][f] = A_BYTES + (sp * 8 + wn * 4 + f) * 1024 + lane * 16;
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The k loop; a wave whose 64 tokens are all past T only loads and syncs.
  auto kloop = [&](auto live_c) {
    constexpr bool LIVE = decltype(live_c)::value;
#pragma unroll
    for (int s0 = 0; s0 < NS - 1; ++s0)
      if (s0 < nk) issue(s0);
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + NS - 2 < nk)
        wait_vmcnt<(NS - 2) * PER_STAGE>();
      else
        wait_vmcnt<0>();
      barrier_only();
      asm volatile("" ::: "memory");
      if (kt + NS - 1 < nk) issue(kt + NS - 1);
      if constexpr (LIVE) {
        const uint8_t* st = smem + (kt % NS) * STAGE;
        u32x4 af[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) af[f] = ld16(st + aoff[f]);
#pragma unroll
        for (int sp = 0; sp < 3; ++sp) {
          u32x4 bfr[4];
#pragma unroll
          for (int f = 0; f < 4; ++f) bfr[f] = ld16(st + boff[sp][f]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[i][j] = mfma_bf16(as_bf16x8(bfr[j]), as_bf16x8(af[i]), acc[i][j]);
        }
      }
      wait_lgkmcnt0();
      asm volatile("" ::: "memory");
    }
  };
  if (tok0 + wm * 64 < T)
    kloop(std::integral_constant<bool, true>{});
  else
    kloop(std::integral_constant<bool, false>{});

  float* zo = zp + (size_t)blockIdx.z * T * kExperts;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = tok0 + wm * 64 + i * 16 + r;
    if (t < T) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        st16(zo + (size_t)t * kExperts + e0 + wn * 64 + j * 16 + 4 * g,
             u32x4{__float_as_uint(acc[i][j][0]), __float_as_uint(acc[i][j][1]),
                   __float_as_uint(acc[i][j][2]), __float_as_uint(acc[i][j][3])});
    }
  }
}

// Maximum of v over the wave, in every lane. DPP steps: neighbours and
// quads (quad permutes), 8 and 16 lanes (half-row and row mirrors), then
// rows 0-1 and 0-3 through the row broadcasts of lanes 15 and 31; lane 63
// ends with the maximum of all 64. A source lane outside the move keeps the
// lane's own value (old = v), which leaves the maximum unchanged.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_max(float v) {
  const int o = __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROWS, 0xF,
                                            false);
  return fmaxf(v, __int_as_float(o));
}

__device__ __forceinline__ float wave_max(float v) {
  v = dpp_max<0xB1>(v);        // quad_perm [1, 0, 3, 2]
  v = dpp_max<0x4E>(v);        // quad_perm [2, 3, 0, 1]
  v = dpp_max<0x141>(v);       // row_half_mirror
  v = dpp_max<0x140>(v);       // row_mirror
  v = dpp_max<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// One wave per token. Lane l holds experts 4l..4l+3. A group of
// 256/n_group experts spans lpg = 64/n_group lanes.
// The logits are the sum of `nparts` partial arrays (stride pstride floats),
// added in order; with zout set the sum is also stored there.
__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ z, int nparts,
                                                     size_t pstride, float* __restrict__ zout,
                                                     const float* __restrict__ bias, int T,
                                                     int n_group, int topk_group, int top_k,
                                                     int32_t* __restrict__ idx,
                                                     float* __restrict__ wout,
                                                     float* __restrict__ sout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;

  const size_t zo = (size_t)t * kExperts + 4 * lane;
  u32x4 zv = ld16(z + zo);
  auto add = [&](const u32x4& o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) zv[i] = __float_as_uint(__uint_as_float(zv[i]) + __uint_as_float(o[i]));
  };
  // partials 1, 2, ... added in order; loaded four at a time so that the
  // loads of a batch are in flight together
  int p = 1;
  for (; p + 4 <= nparts; p += 4) {
    u32x4 o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = ld16(z + (p + q) * pstride + zo);
#pragma unroll
    for (int q = 0; q < 4; ++q) add(o[q]);
  }
  for (; p < nparts; ++p) add(ld16(z + p * pstride + zo));
  if (zout) st16(zout + zo, zv);
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
  // Every lane of a group holds its score, so lane gg * lpg speaks for group gg.
  int rank = 0;
  for (int gg = 0; gg < n_group; ++gg) {
    const float sc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gscore), gg * lpg));
    rank += (sc > gscore || (sc == gscore && gg < grp)) ? 1 : 0;
  }
  uint32_t avail = (rank < topk_group) ? 0xFu : 0u;

  // top_k rounds: the largest remaining key (a wave max), then the lowest
  // expert index holding it: the first lane whose remaining keys reach the
  // max (lane l holds experts 4l .. 4l + 3), its first slot with that key.
  float sum = 0.f, my_s = 0.f;
  int my_i = 0;
  for (int j = 0; j < top_k; ++j) {
    float lmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if ((avail >> i) & 1u) lmax = fmaxf(lmax, key[i]);
    const float m = wave_max(lmax);
    // at least top_k candidates exist, so some lane with candidates left holds m
    const uint64_t hold = __ballot(avail != 0u && lmax == m);
    const int owner = __ffsll((unsigned long long)hold) - 1;
    int first = 3;
#pragma unroll
    for (int i = 3; i >= 0; --i)
      if (((avail >> i) & 1u) && key[i] == m) first = i;
    const int slot = __builtin_amdgcn_readlane(first, owner);
    if (lane == owner) avail &= ~(1u << slot);
    const float sv = (slot == 0) ? s[0] : (slot == 1) ? s[1] : (slot == 2) ? s[2] : s[3];
    const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), owner));
    sum += ws;
    if (lane == j) {
      my_i = 4 * owner + slot;
      my_s = ws;
    }
  }
  if (lane < top_k) {
    idx[(size_t)t * top_k + lane] = my_i;
    wout[(size_t)t * top_k + lane] = my_s / sum;
    if (sout) sout[(size_t)t * top_k + lane] = my_s;
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

int router_small_split(int H) {
  // 16 k per MFMA step x 4 waves per split
  return H % 512 == 0 ? 8 : H % 256 == 0 ? 4 : H % 128 == 0 ? 2 : 1;
}

hipError_t launch_router_logits_split(const void* x, int x_f32, const float* W, float* zp, int T,
                                      int H, int nz, hipStream_t st) {
  // Few tokens: 16x16 tiles, the reduction split over the 4 waves and over
  // nz workgroups, so that enough workgroups stream the router matrix.
  dim3 grid((T + 15) / 16, kExperts / 16, nz);
  if (x_f32)
    router_logits_kernel<float, 1, 4, 1><<<grid, 256, 0, st>>>((const float*)x, W, zp, T, H);
  else
    router_logits_kernel<uint16_t, 1, 4, 1><<<grid, 256, 0, st>>>((const uint16_t*)x, W, zp, T, H);
  return hipGetLastError();
}

int router_ksplit(int T, int H) {
  // Enough workgroups for the 256 CUs (about 512): split the reduction when
  // there are few 256-token tiles, into a power of two that divides H / 32.
  const int tiles = 2 * ((T + kRxBM - 1) / kRxBM);
  const int nk = H / 32;
  int ks = 1;
  while (ks < 16 && tiles * ks < 512 && nk % (2 * ks) == 0) ks *= 2;
  return ks;
}

hipError_t launch_router_x3(const uint16_t* x, const float* W, uint16_t* wsplit, float* zp, int T,
                            int H, int ks, hipStream_t st) {
  router_split_kernel<<<(kExperts * (H / 8) + 255) / 256, 256, 0, st>>>(W, H, wsplit);
  dim3 grid((T + kRxBM - 1) / kRxBM, kExperts / kRxBN, ks);
  router_x3_kernel<<<grid, 512, 0, st>>>(x, wsplit, zp, T, H);
  return hipGetLastError();
}

hipError_t launch_select(const float* z, int nparts, size_t pstride, float* zout, const float* bias,
                         int T, int n_group, int topk_group, int top_k, int32_t* idx, float* w,
                         float* s_sel, hipStream_t st) {
  select_kernel<<<(T + 3) / 4, 256, 0, st>>>(z, nparts, pstride, zout, bias, T, n_group,
                                             topk_group, top_k, idx, w, s_sel);
  return hipGetLastError();
}

}  // namespace beam
