// Token permutation of the Beam MoE block on gfx950: the (token, slot) pairs
// chosen by the router are ordered by expert, stably by token, so that each
// expert's rows are contiguous for the grouped expert GEMMs.
//
// Tokens are processed in chunks of 256 (one workgroup). Inside a chunk a
// 256-bit LDS mask per expert records which tokens chose it; a token never
// chooses the same expert twice, so a pair's rank among the chunk's pairs of
// the same expert is the number of set mask bits below its token. Per-chunk
// counts are scanned per expert across chunks, and the per-expert totals are
// scanned across experts, all with integer arithmetic: the permutation is
// deterministic and stable (ascending token within each expert).
#include "common.h"
#include "internal.h"

namespace beam {

constexpr int kMaskWords = kChunk / 32;  // 8 words of 32 tokens per expert

__device__ __forceinline__ void build_masks(uint32_t* mask, const int32_t* __restrict__ idx, int T,
                                            int k, int chunk) {
  for (int i = threadIdx.x; i < kExperts * kMaskWords; i += 256) mask[i] = 0u;
  __syncthreads();
  const int t = chunk * kChunk + threadIdx.x;
  if (t < T) {
    const uint32_t bit = 1u << (threadIdx.x & 31);
    const int word = threadIdx.x >> 5;
    for (int j = 0; j < k; ++j) {
      const int e = idx[(size_t)t * k + j];
      atomicOr(&mask[e * kMaskWords + word], bit);
    }
  }
  __syncthreads();
}

// chist[c, e] = number of tokens of chunk c that chose expert e.
__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t* __restrict__ idx, int T, int k,
                                                        int32_t* __restrict__ chist) {
  __shared__ uint32_t mask[kExperts * kMaskWords];
  build_masks(mask, idx, T, k, blockIdx.x);
  const int e = threadIdx.x;
  int cnt = 0;
#pragma unroll
  for (int w = 0; w < kMaskWords; ++w) cnt += __popc(mask[e * kMaskWords + w]);
  chist[(size_t)blockIdx.x * kExperts + e] = cnt;
}

// M-tile slots of an expert with n rows. BM rows per slot; with
// BM == kMixedBM the slots hold 256 rows and an expert with more than 256
// rows takes 512-row tiles, two slots each (so its count is even and the
// first slot of each pair starts the tile).
__device__ __forceinline__ int expert_slots(int n, int BM) {
  if (BM != kMixedBM) return (n + BM - 1) / BM;
  return n > 256 ? 2 * ((n + 511) / 512) : (n + 255) / 256;
}

__device__ __forceinline__ int slot_rows(int BM) { return BM == kMixedBM ? 256 : BM; }

// Exclusive prefix sum over the 256 threads of the block.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  __syncthreads();
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  return base + incl - v;
}

// One workgroup, thread e = expert e:
//   cbase[c, e]  = tokens of expert e in chunks before c;
//   counts[e]    = tokens of expert e; offsets = exclusive scan of counts;
//   M-tiles of BM rows per expert (expert_slots), listed expert by expert:
//   tile_e[m] = expert, tile_r[m] = first sorted row; meta[0] = tile count;
//   e_tstart[e], e_ntiles[e] = first M-tile of expert e and its tile count.
__global__ __launch_bounds__(256) void perm_scan_kernel(const int32_t* __restrict__ chist,
                                                        int nchunks, int BM, int e0, int e1,
                                                        int32_t* __restrict__ cbase,
                                                        int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ meta,
                                                        int32_t* __restrict__ tile_e,
                                                        int32_t* __restrict__ tile_r,
                                                        int32_t* __restrict__ e_tstart,
                                                        int32_t* __restrict__ e_ntiles,
                                                        int32_t* __restrict__ counts_out) {
  __shared__ int wsum[4];
  const int e = threadIdx.x;
  int run = 0;
  for (int c = 0; c < nchunks; ++c) {
    const int h = chist[(size_t)c * kExperts + e];
    cbase[(size_t)c * kExperts + e] = run;
    run += h;
  }
  counts[e] = run;
  if (counts_out) counts_out[e] = run;
  const int off = block_exclusive_scan(run, wsum);
  offsets[e] = off;
  if (e == kExperts - 1) offsets[kExperts] = off + run;
  // experts outside [e0, e1) keep their place in the sorted order but get no tiles
  const int mt = (e >= e0 && e < e1) ? expert_slots(run, BM) : 0;
  const int ts = block_exclusive_scan(mt, wsum);
  e_tstart[e] = ts;
  e_ntiles[e] = mt;
  const int sr = slot_rows(BM);
  for (int i = 0; i < mt; ++i) {
    tile_e[ts + i] = e;
    tile_r[ts + i] = off + i * sr;
  }
  if (e == kExperts - 1) meta[0] = ts + mt;
}

// Position of every (token, slot) pair in expert order:
//   pos = offsets[e] + cbase[chunk, e] + (tokens of the chunk below t that chose e).
//   stok[pos] = t, sw[pos] = rsf * w[t, slot], inv[t, slot] = pos.
__global__ __launch_bounds__(256) void perm_scatter_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ w, int T, int k, float rsf,
    const int32_t* __restrict__ cbase, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ stok, float* __restrict__ sw, int32_t* __restrict__ inv) {
  __shared__ uint32_t mask[kExperts * kMaskWords];
  const int c = blockIdx.x;
  build_masks(mask, idx, T, k, c);
  const int t = c * kChunk + threadIdx.x;
  if (t >= T) return;
  const int word = threadIdx.x >> 5;
  const uint32_t below = (1u << (threadIdx.x & 31)) - 1u;
  for (int j = 0; j < k; ++j) {
    const size_t q = (size_t)t * k + j;
    const int e = idx[q];
    int rank = cbase[(size_t)c * kExperts + e];
    for (int ww = 0; ww < word; ++ww) rank += __popc(mask[e * kMaskWords + ww]);
    rank += __popc(mask[e * kMaskWords + word] & below);
    const int pos = offsets[e] + rank;
    stok[pos] = t;
    sw[pos] = rsf * w[q];
    inv[q] = pos;
  }
}

hipError_t launch_perm_hist(const int32_t* idx, int T, int k, int32_t* chist, hipStream_t st) {
  perm_hist_kernel<<<(T + kChunk - 1) / kChunk, 256, 0, st>>>(idx, T, k, chist);
  return hipGetLastError();
}

hipError_t launch_perm_scan(const int32_t* chist, int nchunks, int BM, int32_t* cbase,
                            int32_t* counts, int32_t* offsets, int32_t* meta, int32_t* tile_e,
                            int32_t* tile_r, int32_t* e_tstart, int32_t* e_ntiles,
                            int32_t* counts_out, hipStream_t st, int e0, int e1) {
  perm_scan_kernel<<<1, 256, 0, st>>>(chist, nchunks, BM, e0, e1, cbase, counts, offsets, meta,
                                      tile_e, tile_r, e_tstart, e_ntiles, counts_out);
  return hipGetLastError();
}

// One expert shard's share of the output: out[t] = sum over the slots j
// whose expert lies in [e0, e1) of y_perm[inv[t, j]] (fp32, ascending j; a
// token with no expert in the shard gets zeros). One thread per 8 values.
template <typename OT>
__global__ __launch_bounds__(256) void combine_shard_kernel(const uint16_t* __restrict__ y,
                                                            const int32_t* __restrict__ inv,
                                                            const int32_t* __restrict__ idx,
                                                            int T, int k, int H, int e0, int e1,
                                                            OT* __restrict__ out) {
  const int vpr = H / 8;
  const long long v = (long long)blockIdx.x * 256 + threadIdx.x;
  if (v >= (long long)T * vpr) return;
  const int t = (int)(v / vpr), c = (int)(v % vpr);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int e = idx[(size_t)t * k + j];
    if (e < e0 || e >= e1) continue;
    const u32x4 q = ld16_nt(y + (size_t)inv[(size_t)t * k + j] * H + c * 8);  // read once
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_bits_to_f32(q[i] & 0xffffu);
      acc[2 * i + 1] += bf16_bits_to_f32(q[i] >> 16);
    }
  }
  OT* o = out + (size_t)t * H + c * 8;
  if constexpr (sizeof(OT) == 4) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<u32x4*>(o + 4 * h) =
          u32x4{__float_as_uint(acc[4 * h]), __float_as_uint(acc[4 * h + 1]),
                __float_as_uint(acc[4 * h + 2]), __float_as_uint(acc[4 * h + 3])};
  } else {
    *reinterpret_cast<u32x4*>(o) = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                         pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  }
}

hipError_t launch_combine_shard(const void* y, const int32_t* inv, const int32_t* idx, int T,
                                int k, int H, int e0, int e1, int out_f32, void* out,
                                hipStream_t st) {
  const long long n = (long long)T * (H / 8);
  const int blocks = (int)((n + 255) / 256);
  if (out_f32)
    combine_shard_kernel<float><<<blocks, 256, 0, st>>>((const uint16_t*)y, inv, idx, T, k, H, e0,
                                                        e1, (float*)out);
  else
    combine_shard_kernel<uint16_t><<<blocks, 256, 0, st>>>((const uint16_t*)y, inv, idx, T, k, H,
                                                           e0, e1, (uint16_t*)out);
  return hipGetLastError();
}

// One chunk (T <= 256): the histogram, both scans, the tile list and the
// scatter of the three kernels above in one workgroup, with the same results
// (the chunk's base per expert is 0).
__global__ __launch_bounds__(256) void perm_single_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ w, int T, int k, float rsf, int BM,
    int e0, int e1, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ meta, int32_t* __restrict__ tile_e, int32_t* __restrict__ tile_r,
    int32_t* __restrict__ e_tstart, int32_t* __restrict__ e_ntiles, int32_t* __restrict__ counts_out,
    int32_t* __restrict__ stok, float* __restrict__ sw, int32_t* __restrict__ inv) {
  __shared__ uint32_t mask[kExperts * kMaskWords];
  __shared__ int wsum[4];
  __shared__ int eoff[kExperts];
  build_masks(mask, idx, T, k, 0);
  const int e = threadIdx.x;
  int run = 0;
#pragma unroll
  for (int ww = 0; ww < kMaskWords; ++ww) run += __popc(mask[e * kMaskWords + ww]);
  counts[e] = run;
  if (counts_out) counts_out[e] = run;
  const int off = block_exclusive_scan(run, wsum);
  offsets[e] = off;
  if (e == kExperts - 1) offsets[kExperts] = off + run;
  const int mt = (e >= e0 && e < e1) ? expert_slots(run, BM) : 0;
  const int ts = block_exclusive_scan(mt, wsum);
  e_tstart[e] = ts;
  e_ntiles[e] = mt;
  const int sr = slot_rows(BM);
  for (int i = 0; i < mt; ++i) {
    tile_e[ts + i] = e;
    tile_r[ts + i] = off + i * sr;
  }
  if (e == kExperts - 1) meta[0] = ts + mt;
  eoff[e] = off;
  __syncthreads();
  const int t = threadIdx.x;
  if (t >= T) return;
  const int word = t >> 5;
  const uint32_t below = (1u << (t & 31)) - 1u;
  for (int j = 0; j < k; ++j) {
    const size_t q = (size_t)t * k + j;
    const int ex = idx[q];
    int rank = 0;
    for (int ww = 0; ww < word; ++ww) rank += __popc(mask[ex * kMaskWords + ww]);
    rank += __popc(mask[ex * kMaskWords + word] & below);
    const int pos = eoff[ex] + rank;
    stok[pos] = t;
    sw[pos] = rsf * w[q];
    inv[q] = pos;
  }
}

hipError_t launch_perm_single(const int32_t* idx, const float* w, int T, int k, float rsf, int BM,
                              int32_t* counts, int32_t* offsets, int32_t* meta, int32_t* tile_e,
                              int32_t* tile_r, int32_t* e_tstart, int32_t* e_ntiles,
                              int32_t* counts_out, int32_t* stok, float* sw, int32_t* inv,
                              hipStream_t st, int e0, int e1) {
  if (T > kChunk) return hipErrorInvalidValue;
  perm_single_kernel<<<1, 256, 0, st>>>(idx, w, T, k, rsf, BM, e0, e1, counts, offsets, meta,
                                        tile_e, tile_r, e_tstart, e_ntiles, counts_out, stok, sw,
                                        inv);
  return hipGetLastError();
}

hipError_t launch_perm_scatter(const int32_t* idx, const float* w, int T, int k, float rsf,
                               const int32_t* cbase, const int32_t* offsets, int32_t* stok,
                               float* sw, int32_t* inv, hipStream_t st) {
  perm_scatter_kernel<<<(T + kChunk - 1) / kChunk, 256, 0, st>>>(idx, w, T, k, rsf, cbase,
                                                                  offsets, stok, sw, inv);
  return hipGetLastError();
}

}  // namespace beam
