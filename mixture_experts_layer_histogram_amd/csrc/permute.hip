// Dispatch: expert histogram -> prefix scan -> stable permutation -> capacity
// -> gather of token rows into expert order.
//
// [G] "Load balancing and expert capacity": the example counts the tokens per
// expert (a histogram over the chosen experts) and hands each expert the
// tokens that chose it.  [X] "Deep dive" / "Technical insight": dispatch sends
// every token to the holder of its expert; capacity bounds the tokens an
// expert takes.  [N] "Load balancing" item 2: at most C * N / E tokens per
// expert, the overflow skips the experts.
//
// Priority: slots are ranked in "priority order" i = 0 .. N k - 1: slot order
// (i = s = t k + j) or choice order (i = j N + t: every first choice before
// any second choice).  Ranks, the capacity cut and the row order inside an
// expert all follow i.  Layout: packed rows (offsets = scan of kept counts)
// or fixed [E, C] buffers (offsets = e C; rows past an expert's kept count
// get perm = -1 and, when x_perm is written, zero rows).
//
// Three passes, no atomics on values that decide positions:
//   1. hist_rank   : per block of 1024 slots, the stable rank of every slot
//                    among the block's slots of the same expert, and the
//                    block's per-expert counts [blocks][E].
//   2. scan        : per expert, the exclusive prefix of the block counts (the
//                    rank base of each block), the total count, the kept
//                    count min(count, C), offsets (exclusive scan over
//                    experts) and the drop count.
//   3. scatter     : global rank = base + local rank; kept slots get their
//                    position offsets[e] + rank, write perm/slot_pos and copy
//                    their token row into x_perm with 16-byte loads/stores.
//                    Without x_perm (the expert GEMM then reads the token
//                    rows through perm) only the indices are written.
#include "moe_internal.h"

namespace moe {

constexpr int kHistWaves = 4;

// slot of priority index i, and priority index of slot s
__device__ __forceinline__ int slot_of(int i, int N, int k, bool choice) { return choice ? (i % N) * k + i / N : i; }
__device__ __forceinline__ int index_of(int s, int N, int k, bool choice) { return choice ? (s % k) * N + s / k : s; }
constexpr int kHistChunks = kHistSlotsPerBlock / (64 * kHistWaves);   // 64-slot chunks per wave

// Pass 1.  Wave w of block b owns slots [b*1024 + w*256, +256) and walks them
// in four chunks of 64.  Lanes holding the same expert are found with eight
// ballots (one per bit of the expert id); a lane's rank in the chunk is the
// number of lower lanes in its match set.  The running per-wave count of each
// expert lives in LDS.
__global__ __launch_bounds__(256) void hist_rank_kernel(const int32_t* __restrict__ topk_idx,
                                                        int n_slots, int E, int nblk,
                                                        int32_t* __restrict__ local_rank,
                                                        int32_t* __restrict__ block_counts, int N, int k,
                                                        int choice) {
  __shared__ int cnt[kHistWaves][kMaxExperts];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < kHistWaves * kMaxExperts; i += blockDim.x) (&cnt[0][0])[i] = 0;
  __syncthreads();

  const int base = blockIdx.x * kHistSlotsPerBlock + wave * 64 * kHistChunks;
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank[kHistChunks], eid[kHistChunks];
#pragma unroll
  for (int ch = 0; ch < kHistChunks; ++ch) {
    const int i = base + ch * 64 + lane;
    const int e = i < n_slots ? topk_idx[slot_of(i, N, k, choice)] : -1;
    uint64_t match = __ballot(e >= 0);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const int on = (e >> bit) & 1;
      const uint64_t bb = __ballot(on);
      match &= on ? bb : ~bb;
    }
    const int r = __popcll(match & lower);
    const int before = e >= 0 ? cnt[wave][e] : 0;
    __builtin_amdgcn_wave_barrier();
    if (e >= 0 && r == 0) cnt[wave][e] = before + __popcll(match);
    __builtin_amdgcn_wave_barrier();
    rank[ch] = before + r;
    eid[ch] = e;
  }
  __syncthreads();
  // exclusive prefix over waves (in wave order) and block totals
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int a = 0;
#pragma unroll
    for (int w = 0; w < kHistWaves; ++w) {
      const int c = cnt[w][e];
      cnt[w][e] = a;
      a += c;
    }
    block_counts[(size_t)blockIdx.x * E + e] = a;
  }
  __syncthreads();
#pragma unroll
  for (int ch = 0; ch < kHistChunks; ++ch) {
    const int i = base + ch * 64 + lane;
    if (i < n_slots) local_rank[slot_of(i, N, k, choice)] = cnt[wave][eid[ch]] + rank[ch];
  }
}

// Pass 2 (one workgroup).  Thread e walks expert e's block counts in block
// order (the threads of a wave read one block's counts side by side); then a
// workgroup scan over experts gives the offsets.
__global__ __launch_bounds__(256) void dispatch_scan_kernel(int32_t* __restrict__ block_counts,
                                                            int nblk, int E, int capacity, int padded,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int64_t* __restrict__ drop_count) {
  __shared__ int wave_tot[4];
  __shared__ long long wave_drop[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int kept = 0;
  long long drop = 0;
  if (tid < E) {
    int a = 0;
    int32_t* col = block_counts + tid;
    for (int b0 = 0; b0 < nblk; b0 += 16) {   // 16 loads in flight, then the running sum in order
      int c[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) c[j] = b0 + j < nblk ? col[(size_t)(b0 + j) * E] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (b0 + j < nblk) col[(size_t)(b0 + j) * E] = a;
        a += c[j];
      }
    }
    counts[tid] = a;
    kept = a < capacity ? a : capacity;
    drop = (long long)(a - kept);
  }
  // inclusive scan of `kept` within the wave
  int incl = kept;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  long long dsum = drop;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) dsum += __shfl_xor(dsum, off);
  if (lane == 63) wave_tot[wave] = incl;
  if (lane == 0) wave_drop[wave] = dsum;
  __syncthreads();
  int prefix = 0;
  for (int w = 0; w < wave; ++w) prefix += wave_tot[w];
  if (tid < E) offsets[tid] = padded ? tid * capacity : prefix + incl - kept;
  if (tid == 0) {
    int tot = 0;
    long long dt = 0;
    for (int w = 0; w < 4; ++w) { tot += wave_tot[w]; dt += wave_drop[w]; }
    offsets[E] = padded ? E * capacity : tot;
    if (drop_count) *drop_count = dt;
  }
}

// Pass 3.  One wavefront per slot; row copies use 16-byte accesses when the
// row size allows it.
__global__ __launch_bounds__(256) void scatter_gather_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ local_rank,
    const int32_t* __restrict__ rank_base, const int32_t* __restrict__ offsets, int n_slots, int k,
    int nblk, int E, int capacity, const char* __restrict__ x, size_t row_bytes, int32_t* __restrict__ perm,
    int32_t* __restrict__ slot_pos, char* __restrict__ x_perm, int N, int choice) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + wave;
  if (s >= n_slots) return;
  const int e = topk_idx[s];
  const int blk = index_of(s, N, k, choice) / kHistSlotsPerBlock;
  const int r = rank_base[(size_t)blk * E + e] + local_rank[s];
  if (r >= capacity) {
    if (lane == 0) slot_pos[s] = -1;
    return;
  }
  const int pos = offsets[e] + r;
  if (lane == 0) {
    perm[pos] = s;
    slot_pos[s] = pos;
  }
  const char* src = x + (size_t)(s / k) * row_bytes;
  char* dst = x_perm + (size_t)pos * row_bytes;
  if ((row_bytes & 15) == 0) {
    for (size_t i = (size_t)lane * 16; i < row_bytes; i += 64 * 16)
      *reinterpret_cast<uint4*>(dst + i) = *reinterpret_cast<const uint4*>(src + i);
  } else {
    for (size_t i = (size_t)lane * 2; i < row_bytes; i += 64 * 2)
      *reinterpret_cast<uint16_t*>(dst + i) = *reinterpret_cast<const uint16_t*>(src + i);
  }
}

// Pass 3 without the row copy: one thread per slot.
__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ topk_idx,
                                                      const int32_t* __restrict__ local_rank,
                                                      const int32_t* __restrict__ rank_base,
                                                      const int32_t* __restrict__ offsets, int n_slots,
                                                      int nblk, int E, int capacity, int32_t* __restrict__ perm,
                                                      int32_t* __restrict__ slot_pos, int N, int k, int choice) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n_slots) return;
  const int e = topk_idx[s];
  const int blk = index_of(s, N, k, choice) / kHistSlotsPerBlock;
  const int r = rank_base[(size_t)blk * E + e] + local_rank[s];
  if (r >= capacity) {
    slot_pos[s] = -1;
    return;
  }
  const int pos = offsets[e] + r;
  perm[pos] = s;
  slot_pos[s] = pos;
}

// Padded layout: rows of expert e past its kept count get perm = -1 and, when
// x_perm is written, a zero row.  One wavefront per buffer row.
__global__ __launch_bounds__(256) void pad_rows_kernel(const int32_t* __restrict__ counts, int E, int capacity,
                                                       int32_t* __restrict__ perm, char* __restrict__ x_perm,
                                                       size_t row_bytes) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long r = (long long)blockIdx.x * 4 + wave;
  if (r >= (long long)E * capacity) return;
  const int e = (int)(r / capacity), j = (int)(r % capacity);
  const int kept = min(counts[e], capacity);
  if (j < kept) return;
  if (lane == 0) perm[r] = -1;
  if (x_perm == nullptr) return;
  char* dst = x_perm + (size_t)r * row_bytes;
  if ((row_bytes & 15) == 0) {
    for (size_t i = (size_t)lane * 16; i < row_bytes; i += 64 * 16) *reinterpret_cast<uint4*>(dst + i) = uint4{0, 0, 0, 0};
  } else {
    for (size_t i = (size_t)lane * 2; i < row_bytes; i += 64 * 2) *reinterpret_cast<uint16_t*>(dst + i) = 0;
  }
}

// All three passes in one workgroup, for at most kHistSlotsPerBlock slots with
// the packed layout and no row copy (decode batches: three launches become
// one).  Pass 1 is hist_rank_kernel's for the single block; its counts are the
// expert totals, so pass 2 is the scan over experts and every block base is 0;
// pass 3 places each slot from the rank it still holds in registers.  Ranks,
// offsets and positions are the ones the three-kernel path computes.
__global__ __launch_bounds__(256) void dispatch_small_kernel(const int32_t* __restrict__ topk_idx, int n_slots,
                                                             int E, int capacity, int N, int k, int choice,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                             int32_t* __restrict__ slot_pos,
                                                             int64_t* __restrict__ drop_count) {
  __shared__ int cnt[kHistWaves][kMaxExperts];
  __shared__ int off[kMaxExperts];
  __shared__ int wave_tot[kHistWaves];
  __shared__ long long wave_drop[kHistWaves];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < kHistWaves * kMaxExperts; i += blockDim.x) (&cnt[0][0])[i] = 0;
  __syncthreads();
  // pass 1: stable rank of each slot among the slots of its expert (ballot match per 64-slot chunk)
  const int base = wave * 64 * kHistChunks;
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank[kHistChunks], eid[kHistChunks];
#pragma unroll
  for (int ch = 0; ch < kHistChunks; ++ch) {
    const int i = base + ch * 64 + lane;
    const int e = i < n_slots ? topk_idx[slot_of(i, N, k, choice)] : -1;
    uint64_t match = __ballot(e >= 0);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const int on = (e >> bit) & 1;
      const uint64_t bb = __ballot(on);
      match &= on ? bb : ~bb;
    }
    const int r = __popcll(match & lower);
    const int before = e >= 0 ? cnt[wave][e] : 0;
    __builtin_amdgcn_wave_barrier();
    if (e >= 0 && r == 0) cnt[wave][e] = before + __popcll(match);
    __builtin_amdgcn_wave_barrier();
    rank[ch] = before + r;
    eid[ch] = e;
  }
  __syncthreads();
  // pass 2: per expert, the exclusive prefix over waves and the total; then the scan over experts
  int kept = 0;
  long long drop = 0;
  if (tid < E) {
    int a = 0;
#pragma unroll
    for (int w = 0; w < kHistWaves; ++w) {
      const int c = cnt[w][tid];
      cnt[w][tid] = a;
      a += c;
    }
    counts[tid] = a;
    kept = a < capacity ? a : capacity;
    drop = (long long)(a - kept);
  }
  int incl = kept;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  long long dsum = drop;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) dsum += __shfl_xor(dsum, o);
  if (lane == 63) wave_tot[wave] = incl;
  if (lane == 0) wave_drop[wave] = dsum;
  __syncthreads();
  int prefix = 0;
  for (int w = 0; w < wave; ++w) prefix += wave_tot[w];
  if (tid < E) {
    off[tid] = prefix + incl - kept;
    offsets[tid] = prefix + incl - kept;
  }
  if (tid == 0) {
    int tot = 0;
    long long dt = 0;
    for (int w = 0; w < kHistWaves; ++w) { tot += wave_tot[w]; dt += wave_drop[w]; }
    offsets[E] = tot;
    if (drop_count) *drop_count = dt;
  }
  __syncthreads();
  // pass 3: positions
#pragma unroll
  for (int ch = 0; ch < kHistChunks; ++ch) {
    const int i = base + ch * 64 + lane;
    if (i >= n_slots) continue;
    const int s = slot_of(i, N, k, choice), e = eid[ch];
    const int r = cnt[wave][e] + rank[ch];
    if (r >= capacity) {
      slot_pos[s] = -1;
    } else {
      const int pos = off[e] + r;
      perm[pos] = s;
      slot_pos[s] = pos;
    }
  }
}

hipError_t launch_permute(const moe_config& c, const Workspace& W, const int32_t* topk_idx,
                          const void* x, int32_t* counts, int32_t* offsets, int32_t* perm,
                          int32_t* slot_pos, int64_t* drop_count, void* x_perm,
                          int32_t* hist_rank, int32_t* hist_blocks, hipStream_t s) {
  const long long n_slots_ll = c.n_tokens * (long long)c.top_k;
  const int n_slots = (int)n_slots_ll;
  const int nblk = W.hist_blocks_n;
  const int E = c.n_experts;
  const int capacity = capacity_of(c);
  const int N = (int)c.n_tokens, k = c.top_k;
  const int choice = c.capacity_priority == MOE_PRIORITY_CHOICE ? 1 : 0;
  const int padded = c.capacity_layout == MOE_CAPACITY_PADDED ? 1 : 0;
  if (n_slots > 0 && n_slots <= kHistSlotsPerBlock && !padded && x_perm == nullptr) {
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(256), 0, s, topk_idx, n_slots, E, capacity, N, k, choice,
                       counts, offsets, perm, slot_pos, drop_count);
    return hipGetLastError();
  }
  if (n_slots > 0) {
    hipLaunchKernelGGL(hist_rank_kernel, dim3(nblk), dim3(256), 0, s, topk_idx, n_slots, E, nblk,
                       hist_rank, hist_blocks, N, k, choice);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(256), 0, s, hist_blocks, n_slots > 0 ? nblk : 0,
                     E, capacity, padded, counts, offsets, drop_count);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || n_slots == 0) return err;
  const size_t esz = c.dtype == MOE_BF16 ? 2 : 4;
  const size_t row_bytes = (size_t)c.d_model * esz;
  if (padded) {
    const long long rows = expert_rows(c);
    if (rows > 0) {
      hipLaunchKernelGGL(pad_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, counts, E, capacity,
                         perm, (char*)x_perm, row_bytes);
      err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
  }
  if (x_perm == nullptr) {
    hipLaunchKernelGGL(scatter_kernel, dim3((n_slots + 255) / 256), dim3(256), 0, s, topk_idx, hist_rank,
                       hist_blocks, offsets, n_slots, nblk, E, capacity, perm, slot_pos, N, k, choice);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(scatter_gather_kernel, dim3((n_slots + 3) / 4), dim3(256), 0, s, topk_idx,
                     hist_rank, hist_blocks, offsets, n_slots, c.top_k, nblk, E, capacity,
                     (const char*)x, row_bytes, perm, slot_pos, (char*)x_perm, N, choice);
  return hipGetLastError();
}

}  // namespace moe
