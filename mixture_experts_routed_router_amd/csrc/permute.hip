// permute.hip -- dispatch permutation into beta-aligned expert segments (moe_permute).
//
// MegaFlux §3.1 / App. A.2: inside each expert the routed assignments keep a stable order by
// source and (token, top-k slot), i.e. the flat entry index t*K + k, and the rows are cut into
// blocks of at most beta rows; each expert's segment therefore starts on a multiple of beta.
//
// From 64 blocks of 256 tokens (16384 tokens) on, while blocks x local experts is at most 16384,
// two index launches, without order-dependent atomics:
//   count   block s: the entries of each local expert among tokens [256 s, 256 s + 256)
//           (LDS counts), one row of the workspace per block;
//   place   block s: the padded segment starts (a block scan over the experts' counts), the
//           entries of each expert in the blocks before s (the earlier workspace rows, summed
//           by all threads into LDS), and each entry's rank among the block's tokens that
//           picked the same expert, read off a 256-bit token mask per expert (a token's K
//           experts are distinct, so each (token, expert) pair is one entry); writes entry_pos
//           and row_token, and -1 in row_token for the padding rows of experts s, s + grid, ...
// Otherwise three index launches:
//   hist    per chunk of 16 tokens, the number of entries of each local expert (LDS counts);
//   scan    one workgroup per local expert: the padded segment start, an exclusive scan of
//           the expert's chunk counts (so each chunk knows where its rows begin), and -1 in
//           row_token for the segment's padding rows;
//   scatter one workgroup per chunk: an entry's rank inside the chunk from a 16-bit token
//           mask per expert; writes entry_pos and row_token.
// Every launch costs about 4.6 us of GPU time even with little to do.  The two-pass form saves
// one, and pays off once the scan's walk over T / 16 chunk counts per expert grows (per call:
// 16.5 us in two passes against 20.8 in three at 32768 tokens and 32 local experts, 16.9
// against 20.2 at 16384 tokens and 128 experts); on shorter batches its place pass, one long chain of loads, barriers and LDS reads per block,
// measured about 1 us slower than the three short passes (4096 tokens, 64 experts).  Past
// 16384 count values, summing the earlier blocks' rows in every block would grow with the
// square of the batch.
// Then, when xp is wanted:
//   copy    each token row of x that has a local entry is read once and written to each of
//           its local rows of xp, 16 bytes per thread (the HBM-bound part); skipped when xp
//           is not wanted (the expert GEMM then reads x rows through row_token itself).
#include "moe_launch.h"

namespace {

constexpr int kChunk = MOE_PERMUTE_CHUNK;  // tokens per chunk
constexpr int kThreads = 256;

// The two-pass form: from this many blocks of kThreads tokens, and at most this many workspace
// values (blocks x local experts), so that no block sums more than 64 of them per thread.
constexpr int kMinTwoPassBlocks = 64;
constexpr int kMaxTwoPassValues = 64 * 256;

// Block s: ws[s * E_loc + l] = entries of local expert l among tokens [256 s, 256 s + 256).
__global__ void __launch_bounds__(kThreads)
permute_count_kernel(const int32_t* __restrict__ ids, int T, int K, int begin, int stride,
                     int E_loc, int32_t* __restrict__ ws) {
    __shared__ int h[256];
    const int tid = threadIdx.x;
    if (tid < E_loc) h[tid] = 0;
    __syncthreads();
    const int t = blockIdx.x * kThreads + tid;
    if (t < T) {
        for (int k = 0; k < K; ++k) {
            const int l = moe_local_index(ids[(size_t)t * K + k], begin, stride, E_loc);
            if (l >= 0) atomicAdd(&h[l], 1);
        }
    }
    __syncthreads();
    if (tid < E_loc) ws[(size_t)blockIdx.x * E_loc + tid] = h[tid];
}

// Block s: rows of the entries of tokens [256 s, 256 s + 256), and the padding rows of the
// experts l = s, s + gridDim.x, ...  The global loads a block needs (the experts' counts, its
// tokens' ids, the earlier blocks' workspace rows) are independent and go out together, before
// any of them is used.
__global__ void __launch_bounds__(kThreads)
permute_place_kernel(const int32_t* __restrict__ ids, int T, int K,
                     const int32_t* __restrict__ counts, int begin, int stride, int E_loc,
                     int beta, const int32_t* __restrict__ ws, int32_t* __restrict__ offsets,
                     int32_t* __restrict__ entry_pos, int32_t* __restrict__ row_token) {
    // token bits per local expert: bit j of mask[l][j / 64] = token 256 s + j picked expert l
    __shared__ __align__(16) unsigned long long mask[256][kThreads / 64];
    __shared__ int off_s[257];
    __shared__ int n_s[256];
    __shared__ int base_s[256];  // entries of expert l in earlier blocks, then + its start
    __shared__ int part[kThreads / MOE_WAVE];
    const int tid = threadIdx.x, lane = moe_lane_id(), wave = tid / MOE_WAVE;
    const int s = blockIdx.x;
    const int t = s * kThreads + tid;

    // the global loads first (counts, this thread's entries, the first 16 of the earlier blocks'
    // workspace values); the barrier below waits for them while the LDS is cleared
    const int n = tid < E_loc ? counts[begin + tid * stride] : 0;
    int lk[MOE_MAX_K];
#pragma unroll
    for (int k = 0; k < MOE_MAX_K; ++k)
        lk[k] = (k < K && t < T) ? ids[(size_t)t * K + k] : -1;
    const int m = s * E_loc;  // earlier workspace values: rows 0 .. s - 1
    constexpr int kBatch = 16;
    int v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = tid + u * kThreads < m ? ws[tid + u * kThreads] : 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) mask[tid][w] = 0ull;
    base_s[tid] = 0;
    __syncthreads();

    // padded segment starts: exclusive block scan of ceil(n / beta) beta
    const int seg = (n + beta - 1) / beta * beta;
    int incl = seg;
#pragma unroll
    for (int d = 1; d < MOE_WAVE; d <<= 1) {
        const int o = __shfl_up(incl, d, MOE_WAVE);
        if (lane >= d) incl += o;
    }
    if (lane == MOE_WAVE - 1) part[wave] = incl;
    // entries of each expert in the earlier blocks, added into LDS
    for (int i0 = 0;;) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (i0 + tid + u * kThreads < m)
                atomicAdd(&base_s[(i0 + tid + u * kThreads) % E_loc], v[u]);
        i0 += kBatch * kThreads;
        if (i0 >= m) break;
        // the next kBatch values, all loads in flight together
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            v[u] = i0 + tid + u * kThreads < m ? ws[i0 + tid + u * kThreads] : 0;
    }
    // token masks
#pragma unroll
    for (int k = 0; k < MOE_MAX_K; ++k) {
        lk[k] = lk[k] >= 0 ? moe_local_index(lk[k], begin, stride, E_loc) : -1;
        if (lk[k] >= 0) atomicOr(&mask[lk[k]][tid >> 6], 1ull << (tid & 63));
    }
    __syncthreads();
    int off = incl - seg, total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / MOE_WAVE; ++w) {
        off += w < wave ? part[w] : 0;
        total += part[w];
    }
    if (tid < E_loc) {
        off_s[tid] = off;
        n_s[tid] = n;
        base_s[tid] += off;  // this thread's own expert: no other thread touches it now
        if (s == 0) offsets[tid] = off;
    }
    if (tid == 0) {
        off_s[E_loc] = total;
        if (s == 0) offsets[E_loc] = total;
    }
    // each entry's rank among the block's tokens that picked its expert: the expert's four
    // mask words in two 16-byte reads
    int rk[MOE_MAX_K];
    {
        const int w = tid >> 6;
        const unsigned long long below = (1ull << (tid & 63)) - 1ull;
#pragma unroll
        for (int k = 0; k < MOE_MAX_K; ++k) {
            rk[k] = 0;
            if (lk[k] >= 0) {
                const ulonglong2 m01 = *reinterpret_cast<const ulonglong2*>(&mask[lk[k]][0]);
                const ulonglong2 m23 = *reinterpret_cast<const ulonglong2*>(&mask[lk[k]][2]);
                const unsigned long long mw[4] = {m01.x, m01.y, m23.x, m23.y};
                int r = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    r += q < w ? __popcll(mw[q]) : q == w ? __popcll(mw[q] & below) : 0;
                rk[k] = r;
            }
        }
    }
    __syncthreads();
    // entry rows: segment start + entries in earlier blocks + rank
    if (t < T) {
#pragma unroll
        for (int k = 0; k < MOE_MAX_K; ++k) {
            if (k < K) {
                const int l = lk[k];
                int p = -1;
                if (l >= 0) {
                    p = base_s[l] + rk[k];
                    row_token[p] = t;
                }
                entry_pos[(size_t)t * K + k] = p;
            }
        }
    }
    // padding rows of this block's experts
    for (int l = s; l < E_loc; l += gridDim.x)
        for (int p = off_s[l] + n_s[l] + tid; p < off_s[l + 1]; p += kThreads) row_token[p] = -1;
}

// Block: 256 tokens = 16 chunks.  ws[c * E_loc + l] = entries of local expert l in chunk c.
__global__ void __launch_bounds__(kThreads)
permute_hist_kernel(const int32_t* __restrict__ ids, int T, int K, int begin, int stride,
                    int E_loc, int n_chunks, int32_t* __restrict__ ws) {
    __shared__ int h[kThreads / kChunk][256];
    const int tid = threadIdx.x;
    for (int i = tid; i < (kThreads / kChunk) * E_loc; i += kThreads) h[i / E_loc][i % E_loc] = 0;
    __syncthreads();
    const int t = blockIdx.x * kThreads + tid;
    if (t < T) {
        for (int k = 0; k < K; ++k) {
            int l = moe_local_index(ids[(size_t)t * K + k], begin, stride, E_loc);
            if (l >= 0) atomicAdd(&h[tid / kChunk][l], 1);
        }
    }
    __syncthreads();
    const int c0 = blockIdx.x * (kThreads / kChunk);
    for (int i = tid; i < (kThreads / kChunk) * E_loc; i += kThreads) {
        int c = c0 + i / E_loc;
        if (c < n_chunks) ws[(size_t)c * E_loc + i % E_loc] = h[i / E_loc][i % E_loc];
    }
}

// Block l: segment start of local expert l, exclusive scan of its chunk counts (in place),
// padding rows of its segment marked -1.
__global__ void __launch_bounds__(kThreads)
permute_scan_kernel(const int32_t* __restrict__ counts, int begin, int stride, int E_loc,
                    int beta, int n_chunks, int32_t* __restrict__ ws,
                    int32_t* __restrict__ offsets, int32_t* __restrict__ row_token) {
    __shared__ int part[kThreads];
    const int l = blockIdx.x;
    const int tid = threadIdx.x;

    // padded start of segment l = sum over j < l of ceil(n_j / beta) * beta
    int s = 0;
    for (int j = tid; j < l; j += kThreads) {
        int n = counts[begin + j * stride];
        s += (n + beta - 1) / beta * beta;
    }
    part[tid] = s;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
        if (tid < w) part[tid] += part[tid + w];
        __syncthreads();
    }
    const int off = part[0];
    const int n_l = counts[begin + l * stride];
    const int seg = (n_l + beta - 1) / beta * beta;
    if (tid == 0) {
        offsets[l] = off;
        if (l == E_loc - 1) offsets[E_loc] = off + seg;
    }
    __syncthreads();

    // exclusive scan over chunks of ws[c][l]; thread tid owns a contiguous run of chunks
    const int per = (n_chunks + kThreads - 1) / kThreads;
    const int c_begin = min(n_chunks, tid * per);
    const int c_end = min(n_chunks, c_begin + per);
    int run = 0;
    for (int c = c_begin; c < c_end; ++c) run += ws[(size_t)c * E_loc + l];
    part[tid] = run;
    __syncthreads();
    // Hillis-Steele inclusive scan of the per-thread sums
    for (int d = 1; d < kThreads; d <<= 1) {
        int add = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += add;
        __syncthreads();
    }
    int base = part[tid] - run;
    for (int c = c_begin; c < c_end; ++c) {
        int v = ws[(size_t)c * E_loc + l];
        ws[(size_t)c * E_loc + l] = base;
        base += v;
    }
    for (int p = off + n_l + tid; p < off + seg; p += kThreads) row_token[p] = -1;
}

// Block c: rows of the entries of tokens [16c, 16c + 16).
__global__ void __launch_bounds__(kThreads)
permute_scatter_kernel(const int32_t* __restrict__ ids, int T, int K, int begin, int stride,
                       int E_loc, const int32_t* __restrict__ ws,
                       const int32_t* __restrict__ offsets, int32_t* __restrict__ entry_pos,
                       int32_t* __restrict__ row_token) {
    __shared__ uint32_t mask[256];
    __shared__ int base[256];
    const int c = blockIdx.x;
    const int tid = threadIdx.x;
    const int t0 = c * kChunk;
    for (int l = tid; l < E_loc; l += kThreads) {
        mask[l] = 0u;
        base[l] = offsets[l] + ws[(size_t)c * E_loc + l];
    }
    __syncthreads();

    // one thread per entry (token j of the chunk, slot k)
    const int j = tid / K;
    const int k = tid - j * K;
    const int t = t0 + j;
    const bool has_entry = j < kChunk && t < T;
    int l = -1;
    if (has_entry) {
        l = moe_local_index(ids[(size_t)t * K + k], begin, stride, E_loc);
        if (l >= 0) atomicOr(&mask[l], 1u << j);
    }
    __syncthreads();
    if (has_entry) {
        int p = -1;
        if (l >= 0) {
            p = base[l] + __popc(mask[l] & ((1u << j) - 1u));
            row_token[p] = t;
        }
        entry_pos[(size_t)t * K + k] = p;
    }
}

// Row copy: block b moves 16-byte chunks [256 s, 256 s + 256) of token t's row (b = t * segs + s)
// to each of the token's local rows.  entry_pos of a token is block-uniform (scalar loads);
// a token with no local entry is not read.
__global__ void __launch_bounds__(kThreads)
permute_copy_kernel(const uint8_t* __restrict__ x, int64_t row_bytes, int T, int K, int segs,
                    const int32_t* __restrict__ entry_pos, uint8_t* __restrict__ xp) {
    const int n16 = (int)(row_bytes / 16);
    const int64_t total = (int64_t)T * segs;
    for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
        const int t = (int)(b / segs);
        const int c = (int)(b - (int64_t)t * segs) * kThreads + threadIdx.x;
        int pos[MOE_MAX_K];
        bool any = false;
#pragma unroll
        for (int k = 0; k < MOE_MAX_K; ++k) {
            pos[k] = k < K ? entry_pos[(int64_t)t * K + k] : -1;
            any |= pos[k] >= 0;
        }
        if (!any || c >= n16) continue;
        const uint4 v = reinterpret_cast<const uint4*>(x + (int64_t)t * row_bytes)[c];
#pragma unroll
        for (int k = 0; k < MOE_MAX_K; ++k)
            if (pos[k] >= 0) reinterpret_cast<uint4*>(xp + (int64_t)pos[k] * row_bytes)[c] = v;
    }
}

}  // namespace

hipError_t moe_launch_permute(const void* x, int64_t row_bytes, int T, int K,
                              const int32_t* ids, const int32_t* counts, int begin, int stride,
                              int E_loc, int beta, int32_t* offsets, int32_t* entry_pos,
                              int32_t* row_token, void* xp, int32_t* ws, hipStream_t stream) {
    const int n_blocks = (T + kThreads - 1) / kThreads;
    if (n_blocks >= kMinTwoPassBlocks && (int64_t)n_blocks * E_loc <= kMaxTwoPassValues) {
        permute_count_kernel<<<n_blocks, kThreads, 0, stream>>>(ids, T, K, begin, stride, E_loc,
                                                                ws);
        permute_place_kernel<<<n_blocks, kThreads, 0, stream>>>(ids, T, K, counts, begin, stride,
                                                                E_loc, beta, ws, offsets,
                                                                entry_pos, row_token);
    } else {
        const int n_chunks = (T + kChunk - 1) / kChunk;
        permute_hist_kernel<<<n_blocks, kThreads, 0, stream>>>(ids, T, K, begin, stride, E_loc,
                                                               n_chunks, ws);
        permute_scan_kernel<<<E_loc, kThreads, 0, stream>>>(counts, begin, stride, E_loc, beta,
                                                             n_chunks, ws, offsets, row_token);
        permute_scatter_kernel<<<n_chunks, kThreads, 0, stream>>>(ids, T, K, begin, stride,
                                                                   E_loc, ws, offsets, entry_pos,
                                                                   row_token);
    }
    if (xp == nullptr) return hipGetLastError();  // indices only: the GEMM gathers x rows
    const int segs = (int)((row_bytes / 16 + kThreads - 1) / kThreads);
    int64_t grid = (int64_t)T * segs;
    if (grid > 65536) grid = 65536;
    permute_copy_kernel<<<(int)grid, kThreads, 0, stream>>>(static_cast<const uint8_t*>(x),
                                                          row_bytes, T, K, segs, entry_pos,
                                                          static_cast<uint8_t*>(xp));
    return hipGetLastError();
}
