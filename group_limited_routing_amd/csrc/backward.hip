// Kernels of the MoE block's backward pass (besides the GEMM modes of the
// DMA variant): the per-token gradient of the routing weights and the input
// rows, the router-weight gradient, the transposed operand copies and the
// grouped weight-gradient GEMM, the transposed weight packing, and the
// load-balancing bias step.
#include "common.h"
#include "internal.h"

namespace beam {

// ---------------------------------------------------------------- expert segments
// Column of expert e's first row in the transposed operand copies: the
// experts' row counts rounded up to a multiple of 32, scanned. pcol[E] is
// the total. One workgroup of kExperts threads.
__global__ __launch_bounds__(kExperts) void segment_cols_kernel(const int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ pcol) {
  __shared__ int32_t sh[kExperts];
  const int e = threadIdx.x;
  const int v = (counts[e] + 31) & ~31;
  sh[e] = v;
  __syncthreads();
  for (int off = 1; off < kExperts; off <<= 1) {
    const int o = e >= off ? sh[e - off] : 0;
    __syncthreads();
    sh[e] += o;
    __syncthreads();
  }
  pcol[e] = sh[e] - v;
  if (e == kExperts - 1) pcol[kExperts] = sh[e];
}

hipError_t launch_segment_cols(const int32_t* counts, int32_t* pcol, hipStream_t st) {
  segment_cols_kernel<<<1, kExperts, 0, st>>>(counts, pcol);
  return hipGetLastError();
}

// Expert whose segment holds column col, or -1 past the last segment (an
// empty expert's segment holds no column).
__device__ __forceinline__ int segment_of(const int32_t* pcol, int col) {
  if (col >= pcol[kExperts]) return -1;
  int lo = 0, hi = kExperts - 1;  // largest e with pcol[e] <= col
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pcol[mid] <= col) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------- transposed rows
// out(h, col) = scale(q) * src[stok[q]][h] for the sorted rows q of every
// expert, col = pcol[e] + q - offsets[e]; the pad columns of each segment are
// zero. out is [H, pcols] in 32-column blocks (element (h, c) at
// ((c / 32) H + h) 32 + c % 32). A workgroup moves 32 columns x 64 rows
// through LDS: reads of 32 source rows (128 B each), one contiguous 4 KB
// write. SCALED: scale(q) = sw[q] (rsf * routing weight); else 1.
template <bool SCALED>
__global__ __launch_bounds__(256) void gather_t_kernel(const uint16_t* __restrict__ src, int H,
                                                       const int32_t* __restrict__ stok,
                                                       const float* __restrict__ sw,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ pcol,
                                                       uint16_t* __restrict__ out) {
  __shared__ float tile[32][65];
  const int col0 = blockIdx.x * 32, h0 = blockIdx.y * 64;
  const int e = segment_of(pcol, col0);
  if (e < 0) return;
  const int n_e = offsets[e + 1] - offsets[e];
  const int q0 = offsets[e] + col0 - pcol[e];  // sorted row of column col0
  const int tid = threadIdx.x;
  // load: thread -> (row j = tid / 8, 8 values at h0 + 8 (tid % 8)); 32 rows
  {
    const int j = tid >> 3, c = (tid & 7) * 8;
    const int q = q0 + j;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (col0 - pcol[e] + j < n_e) {
      const u32x4 d = ld16(src + (size_t)stok[q] * H + h0 + c);
      const float sc = SCALED ? sw[q] : 1.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_bits_to_f32(d[i] & 0xffffu) * sc;
        v[2 * i + 1] = bf16_bits_to_f32(d[i] >> 16) * sc;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[j][c + i] = v[i];
  }
  __syncthreads();
  // store: thread -> (output row h0 + tid / 4, 8 columns at 8 (tid % 4))
  const int hr = tid >> 2, c8 = (tid & 3) * 8;
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(tile[c8 + 2 * i][hr], tile[c8 + 2 * i + 1][hr]);
  st16(out + (((size_t)(col0 >> 5) * H + h0 + hr) << 5) + c8, o);
}

// Zero the pad columns (past each expert's rows) of up to three [N, pcols]
// matrices in 32-column blocks written by the GEMM epilogues: only each
// expert's last block has pads, N contiguous 64-byte rows. One workgroup per
// expert, a thread per 16-byte chunk (chunks holding live columns keep them).
__global__ __launch_bounds__(256) void zero_pads_kernel(uint16_t* a, uint16_t* b, uint16_t* c,
                                                        int N, const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ pcol) {
  const int e = blockIdx.x;
  const int n_e = offsets[e + 1] - offsets[e], live = n_e & 31;
  if (live == 0) return;  // no pads (or no rows at all)
  const size_t blk = (size_t)((pcol[e] + n_e) >> 5) * N * 32;
  for (int q = threadIdx.x; q < N * 4; q += 256) {
    const int c8 = (q & 3) * 8;
    if (c8 + 8 <= live) continue;
    const size_t off = blk + (size_t)(q >> 2) * 32 + c8;
    uint16_t* bufs[3] = {a, b, c};
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      if (!bufs[m]) continue;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (c8 < live) {  // the chunk holds live columns: keep them
        const u32x4 old = ld16(bufs[m] + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int col = c8 + 2 * i;
          v[i] = (col + 1 < live) ? old[i] : (col < live ? (old[i] & 0xffffu) : 0u);
        }
      }
      st16(bufs[m] + off, v);
    }
  }
}

hipError_t launch_gather_t(const uint16_t* src, int H, bool scaled, const int32_t* stok,
                           const float* sw, const int32_t* offsets, const int32_t* pcol,
                           uint16_t* out, int max_blocks, hipStream_t st) {
  dim3 grid(max_blocks, H / 64);
  if (scaled)
    gather_t_kernel<true><<<grid, 256, 0, st>>>(src, H, stok, sw, offsets, pcol, out);
  else
    gather_t_kernel<false><<<grid, 256, 0, st>>>(src, H, stok, sw, offsets, pcol, out);
  return hipGetLastError();
}

hipError_t launch_zero_pads(uint16_t* a, uint16_t* b, uint16_t* c, int N, const int32_t* offsets,
                            const int32_t* pcol, hipStream_t st) {
  zero_pads_kernel<<<kExperts, 256, 0, st>>>(a, b, c, N, offsets, pcol);
  return hipGetLastError();
}

// ---------------------------------------------------------------- per-token gradients
// One workgroup per token. The routing-weight gradient of slot j is
// dw_j = rsf * sum of the nparts partial sums of h . q of its sorted row;
// through the normalisation and the sigmoid,
//   ds_j = (dw_j - sum_i w_i dw_i) / S,  dz_j = ds_j s_j (1 - s_j)
// (S = sum of the chosen scores). dz goes to dz_sorted at the slot's sorted
// row. Then dx[t] = sum_j dx_rows[inv[t, j]] + sum_j dz_j W_r[e_j], in fp32,
// ascending j, rounded to bf16.
__global__ __launch_bounds__(256) void token_grad_kernel(
    const uint16_t* __restrict__ dxr, const int32_t* __restrict__ inv,
    const int32_t* __restrict__ idx, const float* __restrict__ w, const float* __restrict__ s_sel,
    const float* __restrict__ part, int nparts, float rsf, const float* __restrict__ router_w,
    int k, int H, float* __restrict__ dz_sorted, uint16_t* __restrict__ dx) {
  __shared__ float dzs[32];
  __shared__ int pos[32], ex[32];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < 64) {
    // lanes 0..k-1 of the first wave hold one slot each
    const bool on = tid < k;
    const int p = on ? inv[(size_t)t * k + tid] : 0;
    float dw = 0.f;
    if (on)
      for (int i = 0; i < nparts; ++i) dw += part[(size_t)p * nparts + i];
    dw *= rsf;
    const float wj = on ? w[(size_t)t * k + tid] : 0.f;
    const float sj = on ? s_sel[(size_t)t * k + tid] : 0.f;
    float wdw = wj * dw, S = sj;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      wdw += __shfl_xor(wdw, off);
      S += __shfl_xor(S, off);
    }
    if (on) {
      const float ds = (dw - wdw) / S;
      const float dz = ds * sj * (1.f - sj);
      dzs[tid] = dz;
      pos[tid] = p;
      ex[tid] = idx[(size_t)t * k + tid];
      dz_sorted[p] = dz;
    }
  }
  __syncthreads();
  for (int c = tid * 8; c < H; c += 256 * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      const u32x4 q = ld16(dxr + (size_t)pos[j] * H + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += bf16_bits_to_f32(q[i] & 0xffffu);
        acc[2 * i + 1] += bf16_bits_to_f32(q[i] >> 16);
      }
    }
    for (int j = 0; j < k; ++j) {
      const float* wr = router_w + (size_t)ex[j] * H + c;
      const u32x4 a = ld16(wr), b = ld16(wr + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += dzs[j] * __uint_as_float(a[i]);
        acc[4 + i] += dzs[j] * __uint_as_float(b[i]);
      }
    }
    st16(dx + (size_t)t * H + c, u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                       pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])});
  }
}

hipError_t launch_token_grad(const uint16_t* dxr, const int32_t* inv, const int32_t* idx,
                             const float* w, const float* s_sel, const float* part, int nparts,
                             float rsf, const float* router_w, int T, int k, int H,
                             float* dz_sorted, uint16_t* dx, hipStream_t st) {
  token_grad_kernel<<<T, 256, 0, st>>>(dxr, inv, idx, w, s_sel, part, nparts, rsf, router_w, k, H,
                                       dz_sorted, dx);
  return hipGetLastError();
}

// d W_r[e] = sum over expert e's sorted rows q of dz[q] * x[stok[q]] (fp32,
// rows in sorted order). Grid (E, H / 1024); a thread owns 4 columns.
__global__ __launch_bounds__(256) void router_grad_kernel(const uint16_t* __restrict__ x, int H,
                                                          const int32_t* __restrict__ stok,
                                                          const int32_t* __restrict__ offsets,
                                                          const float* __restrict__ dz,
                                                          float* __restrict__ drw) {
  const int e = blockIdx.x, c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const int q1 = offsets[e + 1];
  for (int q = offsets[e]; q < q1; ++q) {
    const float d = dz[q];
    const u32x2 v = *reinterpret_cast<const u32x2*>(x + (size_t)stok[q] * H + c);
    acc[0] += d * bf16_bits_to_f32(v[0] & 0xffffu);
    acc[1] += d * bf16_bits_to_f32(v[0] >> 16);
    acc[2] += d * bf16_bits_to_f32(v[1] & 0xffffu);
    acc[3] += d * bf16_bits_to_f32(v[1] >> 16);
  }
  st16(drw + (size_t)e * H + c, u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                                      __float_as_uint(acc[2]), __float_as_uint(acc[3])});
}

hipError_t launch_router_grad(const uint16_t* x, int H, const int32_t* stok,
                              const int32_t* offsets, const float* dz, float* drw, hipStream_t st) {
  dim3 grid(kExperts, (H + 1023) / 1024);
  router_grad_kernel<<<grid, 256, 0, st>>>(x, H, stok, offsets, dz, drw);
  return hipGetLastError();
}

// ---------------------------------------------------------------- weight-gradient GEMM
// C[e] (M x N, bf16, row-major) = A_e B_e^T, where A_e and B_e are expert e's
// segments of the transposed copies A [M, pcols] and B [N, pcols] in
// 32-column blocks (the reduction runs over the expert's sorted rows; pad
// columns are zero, and one step's operand rows are contiguous). An
// expert with no rows gets a zero matrix. TM x TN tiles, WAVES waves as a
// 2 x (WAVES / 2) grid, operands by DMA into an NS-stage LDS ring of
// 32-column steps (both operands stored like the A tile of the DMA variant:
// row r's 16-byte chunk g at position g ^ ((r >> 1) & 3)).
template <int TM, int TN, int WAVES, int NS, int OCC = 1>
__global__ __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(WAVES / 4 * OCC, WAVES / 4 * OCC)))
void gemm_wgrad_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bm, int M,
                       int N, const int32_t* __restrict__ pcol, uint16_t* __restrict__ C) {
  constexpr int WN = WAVES / 2;                    // waves along N
  constexpr int WTM = TM / 2, WTN = TN / WN;       // wave tile
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int TA = TM * 64, STAGE = (TM + TN) * 64;
  constexpr int AI = TM / 16 / WAVES, BI = TN / 16 / WAVES;  // DMA instructions per wave
  constexpr int PER = AI + BI;
  static_assert(AI >= 1 && BI >= 1 && FM >= 1 && FN >= 1, "tile shape");
  constexpr int CS = TN * 2 + 16;  // staged output row stride in bytes (padded against bank conflicts)
  constexpr int SMEM = NS * STAGE > TM * CS ? NS * STAGE : TM * CS;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
  const int mtn = M / TM, ntn = N / TN;
  // XCD-contiguous numbering: the blocks on one XCD (b % 8) take a contiguous
  // range of tiles, so an expert's tiles, which share operand rows, meet in
  // that XCD's L2. Inside an expert the N-tile runs fastest.
  const int n_tiles = kExperts * mtn * ntn, b = blockIdx.x;
  if (b >= n_tiles) return;
  const int xcd = b & 7, per = n_tiles >> 3, extra = n_tiles & 7;
  const int j = xcd * per + min(xcd, extra) + (b >> 3);
  const int e = j / (mtn * ntn), rem = j % (mtn * ntn);
  const int m0 = (rem / ntn) * TM, n0 = (rem % ntn) * TN;
  const int c0 = pcol[e], nk = (pcol[e + 1] - c0) / 32;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN, r = lane & 15, g = lane >> 4;
  // DMA sources: instruction i of this wave fills rows 16 (wave * AI + i) .. of the tile
  const uint16_t* asrc[AI];
  const uint16_t* bsrc[BI];
  const size_t cb = (size_t)(c0 >> 5);  // first 32-column block of the segment
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = (wave * AI + i) * 16 + (lane >> 2);
    asrc[i] = A + ((cb * M + m0 + row) << 5) + (((lane & 3) ^ ((row >> 1) & 3)) * 8);
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int row = (wave * BI + i) * 16 + (lane >> 2);
    bsrc[i] = Bm + ((cb * N + n0 + row) << 5) + (((lane & 3) ^ ((row >> 1) & 3)) * 8);
  }
  auto issue = [&](int kt) {
    uint8_t* st = smem + (kt % NS) * STAGE;
#pragma unroll
    for (int i = 0; i < AI; ++i)
      dma16(asrc[i] + ((size_t)kt * M << 5), st + (wave * AI + i) * 1024);
#pragma unroll
    for (int i = 0; i < BI; ++i)
      dma16(bsrc[i] + ((size_t)kt * N << 5), st + TA + (wave * BI + i) * 1024);
  };
  int aoff[FM], boff[FN];
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int row = wm * WTM + f * 16 + r;
    aoff[f] = row * 64 + ((g ^ ((row >> 1) & 3)) << 4);
  }
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    const int row = wn * WTN + f * 16 + r;
    boff[f] = TA + row * 64 + ((g ^ ((row >> 1) & 3)) << 4);
  }
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) acc[i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0)
    if (s0 < nk) issue(s0);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt done for this wave (at most the later issued stages outstanding) ...
    if (kt + NS - 2 < nk)
      wait_vmcnt<(NS - 2) * PER>();
    else
      wait_vmcnt<0>();
    barrier_only();  // ... and for every wave; all reads of kt - 1 retired
    asm volatile("" ::: "memory");
    if (kt + NS - 1 < nk) issue(kt + NS - 1);
    const uint8_t* st = smem + (kt % NS) * STAGE;
    u32x4 af[FM], bfr[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) bfr[f] = ld16(st + boff[f]);
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = ld16(st + aoff[i]);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jn = 0; jn < FN; ++jn)
        acc[i][jn] = mfma_bf16(as_bf16x8(bfr[jn]), as_bf16x8(af[i]), acc[i][jn]);
    wait_lgkmcnt0();
    asm volatile("" ::: "memory");
  }
  // The output tile goes through LDS (over the drained ring) so that global stores
  // are whole 16-byte chunks of contiguous rows. Lane (r, g) of fragment
  // (i, jn) holds tile row WTM wm + 16 i + r, columns WTN wn + 16 jn + 4 g .. + 3.
  __syncthreads();  // every wave is past its last read of the ring
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = wm * WTM + i * 16 + r;
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) {
      const int col = wn * WTN + jn * 16 + 4 * g;
      const f32x4 v = acc[i][jn];
      *reinterpret_cast<u32x2*>(smem + row * CS + col * 2) =
          u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
  }
  __syncthreads();
  uint16_t* Ce = C + (size_t)e * M * N + (size_t)m0 * N + n0;
  constexpr int CPR = TN / 8;  // 16-byte chunks per tile row
  static_assert(TM * CPR % (WAVES * 64) == 0, "whole copy rounds");
#pragma unroll
  for (int it = 0; it < TM * CPR / (WAVES * 64); ++it) {
    const int q = tid + it * WAVES * 64, row = q / CPR, c = q % CPR;
    st16(Ce + (size_t)row * N + c * 8, ld16(smem + row * CS + c * 16));
  }
}

hipError_t launch_wgrad(const uint16_t* A, const uint16_t* B, int M, int N, const int32_t* pcol,
                        uint16_t* C, hipStream_t st) {
  if (M % 256 || N % 256) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)kExperts * (M / 256) * (N / 256);
  gemm_wgrad_kernel<256, 256, 8, 3><<<blocks, 512, 0, st>>>(A, B, M, N, pcol, C);
  return hipGetLastError();
}

// ---------------------------------------------------------------- transposed packing
// Row-major [rows, cols] bf16 matrices to the packed fragment layout of their
// transposes ([cols, rows], the reduction along the source rows). A
// workgroup transposes a 64 x 64 block through LDS: coalesced 128-byte
// source rows in, eight 1 KB fragment blocks (4 row blocks x 2 k-steps) out.
__global__ __launch_bounds__(256) void pack_t_kernel(const uint16_t* __restrict__ src,
                                                     uint16_t* __restrict__ dst, int rows,
                                                     int cols) {
  __shared__ uint16_t tile[64][66];
  const int e = blockIdx.z;
  const int k0 = blockIdx.y * 64, c0 = blockIdx.x * 64;  // source rows (k), source columns
  const uint16_t* S = src + (size_t)e * rows * cols;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int q = tid + 256 * it, rr = q >> 3, cc = (q & 7) * 8;
    const u32x4 v = ld16(S + (size_t)(k0 + rr) * cols + c0 + cc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[rr][cc + 2 * i] = (uint16_t)(v[i] & 0xffffu);
      tile[rr][cc + 2 * i + 1] = (uint16_t)(v[i] >> 16);
    }
  }
  __syncthreads();
  // transposed matrix: row R = c0 + 16 rb + l % 16, k = k0 + 32 ks + 8 (l / 16) .. + 7
  const int ksteps = rows / 32;
  uint16_t* D = dst + (size_t)e * rows * cols;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int q = tid + 256 * it;  // 512 chunks: (rb, ks, lane)
    const int l = q & 63, ks = (q >> 6) & 1, rb = q >> 7;
    const int cl = rb * 16 + (l & 15), kl = ks * 32 + 8 * (l >> 4);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = (uint32_t)tile[kl + 2 * i][cl] | ((uint32_t)tile[kl + 2 * i + 1][cl] << 16);
    const size_t blk = (size_t)((c0 >> 4) + rb) * ksteps + (k0 >> 5) + ks;
    st16(D + blk * 512 + l * 8, o);
  }
}

hipError_t launch_pack_t(const void* src, void* dst, int E, int rows, int cols, hipStream_t st) {
  dim3 grid(cols / 64, rows / 64, E);
  pack_t_kernel<<<grid, 256, 0, st>>>((const uint16_t*)src, (uint16_t*)dst, rows, cols);
  return hipGetLastError();
}

// ---------------------------------------------------------------- bias step
// b_e += gamma * sign(mean load - load_e); the sign is taken exactly, from
// load_e * E against the total load (64-bit integers).
__global__ __launch_bounds__(kExperts) void bias_step_kernel(float* __restrict__ bias,
                                                             const int32_t* __restrict__ counts,
                                                             float gamma) {
  __shared__ long long sh[kExperts];
  const int e = threadIdx.x;
  const long long c = counts[e];
  sh[e] = c;
  __syncthreads();
  for (int off = kExperts / 2; off >= 1; off >>= 1) {
    if (e < off) sh[e] += sh[e + off];
    __syncthreads();
  }
  const long long total = sh[0], mine = c * kExperts;
  const float sg = mine < total ? 1.f : (mine > total ? -1.f : 0.f);
  bias[e] = bias[e] + gamma * sg;
}

hipError_t launch_bias_step(float* bias, const int32_t* counts, float gamma, hipStream_t st) {
  bias_step_kernel<<<1, kExperts, 0, st>>>(bias, counts, gamma);
  return hipGetLastError();
}

}  // namespace beam
