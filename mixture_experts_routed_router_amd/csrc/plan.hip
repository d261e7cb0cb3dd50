// plan.hip -- skew-balancing plan over logical rank partitions + block table (moe_plan).
//
// MoonEP routing flow ("Same data, summed per rank" and "The greedy balance, step by step"):
// a rank's surplus is its experts' entries minus its capacity S*K.  A single move brings the
// rank furthest below capacity back to exactly zero, taking everything it lacks from the rank
// furthest above; that donor may fall below capacity itself and is then topped up by a later
// move.  The donor pays with its own experts, largest remaining first, split where the need
// runs out.  MegaFlux §3.1 / App. A.2: the plan keeps every selection; each
// expert's rows are cut into blocks of at most beta rows in the expert's stable order.
//
// One workgroup.  The greedy is sequential by nature (at most P-1 rank moves, each a few
// slices) and runs in wave 0: lane r holds rank r's surplus in a register, and lane i the
// remaining entries of experts i, i+64, ... (E_loc <= 256).  Every arg-min / arg-max is one
// branch-free reduction of 64-bit (value, index) keys over the wave, under total orders
// (value, then lowest id), so ties resolve exactly as stated in moe.h; lanes that do not
// compete hold the losing key.  The slice counts sit in LDS in table order (rank-major), so
// the block table is emitted by all threads from a scan of per-slice block counts with
// consecutive threads reading consecutive slices; each block is then written by its own thread.
#include "moe_launch.h"
#include "moe_wave.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxSlices = 4096;  // E_loc * P

__global__ void __launch_bounds__(kThreads)
plan_kernel(const int32_t* __restrict__ counts, int begin, int stride, int E_loc, int P,
            int beta, int32_t* __restrict__ q_out, int32_t* __restrict__ moves,
            int32_t* __restrict__ n_moves, int max_moves, int32_t* __restrict__ blocks,
            int32_t* __restrict__ n_blocks, int max_blocks, int32_t* __restrict__ err_word) {
    __shared__ int n_s[256];
    __shared__ int off_s[257];
    // slice (l, r) = the rows of local expert l that rank r computes, kept in table order
    // s = r * E_loc + l: q_s = its row count, start_s = its first row
    __shared__ int q_s[kMaxSlices];
    __shared__ int start_s[kMaxSlices];
    __shared__ int boff_s[kMaxSlices];  // first block of each slice
    __shared__ int part[kThreads / MOE_WAVE];
    __shared__ int err_s;

    const int tid = threadIdx.x;
    const int lane = moe_lane_id();
    const int G = E_loc / P;
    const int S = E_loc * P;

    for (int l = tid; l < E_loc; l += kThreads) n_s[l] = counts[begin + l * stride];
    for (int i = tid; i < S; i += kThreads) q_s[i] = 0;
    if (tid == 0) err_s = 0;
    __syncthreads();

    if (tid < MOE_WAVE) {
        // padded segment starts (same layout as moe_permute) and N, by a wave scan
        int padded[4], raw = 0, pad_sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int l = lane * 4 + j;
            int n = l < E_loc ? n_s[l] : 0;
            padded[j] = (n + beta - 1) / beta * beta;
            pad_sum += padded[j];
            raw += n;
        }
        int incl = pad_sum;
#pragma unroll
        for (int d = 1; d < MOE_WAVE; d <<= 1) {
            int o = __shfl_up(incl, d, MOE_WAVE);
            if (lane >= d) incl += o;
        }
        int run = incl - pad_sum;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int l = lane * 4 + j;
            if (l < E_loc) off_s[l] = run;
            run += padded[j];
        }
        if (lane == MOE_WAVE - 1) off_s[E_loc] = incl;
        const int N = moe_wave_sum_i32(raw);

        // surplus of rank `lane`
        int d = 0;
        if (lane < P) {
            int load = 0;
            for (int l = lane * G; l < (lane + 1) * G; ++l) load += n_s[l];
            d = load - (N / P + (lane < N % P ? 1 : 0));
        }
        // remaining (not yet moved) entries of local expert lane + 64 j, in registers
        int rem[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) rem[j] = lane + 64 * j < E_loc ? n_s[lane + 64 * j] : 0;

        // The greedy runs in uniform control flow: every search is a branch-free reduction of
        // 64-bit (value, index) keys over the whole wave (ranks >= P and experts outside the
        // donor hold the losing key), so the rank min / max searches of one step overlap.
        int nm = 0, err = 0;
        for (int iter = 0; iter <= P; ++iter) {
            const int64_t kmin = wave_best_key<false>(lane < P ? moe_wave::min_key(d, lane) : INT64_MAX);
            const int64_t kmax = wave_best_key<true>(lane < P ? moe_wave::max_key(d, lane) : INT64_MIN);
            const int mn = moe_wave::key_value(kmin);
            if (mn >= 0) break;
            if (iter == P) {  // cannot happen: each move settles one rank for good
                err |= 4;
                break;
            }
            const int recv = moe_wave::min_key_index(kmin), donor = moe_wave::max_key_index(kmax);
            int need = -mn;
            if (lane == donor) d -= need;
            if (lane == recv) d = 0;
            const int e0 = donor * G, e1 = e0 + G;
            for (int sl = 0; need > 0; ++sl) {
                // donor's own expert with the most remaining entries (lowest id on ties)
                int64_t kb = INT64_MIN;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int l = lane + 64 * j;
                    if (l >= e0 && l < e1 && rem[j] > 0) {
                        const int64_t c = moe_wave::max_key(rem[j], l);
                        kb = c > kb ? c : kb;
                    }
                }
                kb = wave_best_key<true>(kb);
                const int bv = moe_wave::key_value(kb);
                const int bl = moe_wave::max_key_index(kb);
                if (kb == INT64_MIN || bv <= 0 || sl > G) {  // cannot happen: a donor covers its move
                    err |= 4;
                    break;
                }
                const int take = bv < need ? bv : need;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (bl == lane + 64 * j) rem[j] -= take;
                if (lane == 0) {
                    atomicAdd(&q_s[recv * E_loc + bl], take);  // no return value: no wait
                    if (nm < max_moves) {
                        const int4 mv = make_int4(donor, recv, bl, take);
                        *reinterpret_cast<int4*>(moves + 4 * nm) = mv;
                    }
                }
                ++nm;
                need -= take;
            }
            if (err) break;
        }
        if (nm > max_moves) err |= 2;
        // leftovers stay with the owner
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int l = lane + 64 * j;
            if (l < E_loc) atomicAdd(&q_s[(l / G) * E_loc + l], rem[j]);
        }
        if (lane == 0) {
            *n_moves = nm < max_moves ? nm : max_moves;
            err_s = err;
        }
    }
    __syncthreads();

    // q output [E_loc, P]; first row of slice (l, r): segment start + rows of expert l taken
    // by lower ranks
    for (int i = tid; i < S; i += kThreads) {
        const int r = i / E_loc, l = i - r * E_loc;
        q_out[l * P + r] = q_s[i];
    }
    for (int l = tid; l < E_loc; l += kThreads) {
        int acc = off_s[l];
        for (int r = 0; r < P; ++r) {
            start_s[r * E_loc + l] = acc;
            acc += q_s[r * E_loc + l];
        }
    }
    __syncthreads();

    // blocks per slice in table order; thread owns a run of slices
    const int per = (S + kThreads - 1) / kThreads;
    const int s_begin = min(S, tid * per);
    const int s_end = min(S, s_begin + per);
    int cnt = 0;
    for (int s = s_begin; s < s_end; ++s) cnt += (q_s[s] + beta - 1) / beta;
    // exclusive scan of the per-thread block counts: within each wave by shuffles, across
    // the four waves through LDS
    int incl = cnt;
#pragma unroll
    for (int dd = 1; dd < MOE_WAVE; dd <<= 1) {
        const int o = __shfl_up(incl, dd, MOE_WAVE);
        if (lane >= dd) incl += o;
    }
    const int wave = tid / MOE_WAVE;
    if (lane == MOE_WAVE - 1) part[wave] = incl;
    __syncthreads();
    int b = incl - cnt, total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / MOE_WAVE; ++w) {
        b += w < wave ? part[w] : 0;
        total += part[w];
    }
    // each slice's first block; then one thread per block finds its slice by a binary search
    // (a slice may hold many blocks: walking them per slice serialised a wave on its largest)
    for (int s = s_begin; s < s_end; ++s) {
        boff_s[s] = b;
        b += (q_s[s] + beta - 1) / beta;
    }
    __syncthreads();
    const int n_emit = total < max_blocks ? total : max_blocks;
    int top = 1;
    while (top * 2 <= S) top *= 2;
    for (int bb = tid; bb < n_emit; bb += kThreads) {
        int s = 0;  // last slice whose first block is <= bb: the slice holding block bb
        for (int step = top; step > 0; step >>= 1)
            if (s + step < S && boff_s[s + step] <= bb) s += step;
        const int r = s / E_loc, l = s - r * E_loc;
        const int j = bb - boff_s[s];
        const int take = q_s[s];
        const int rows = take - j * beta < beta ? take - j * beta : beta;
        *reinterpret_cast<int4*>(blocks + 4 * bb) = make_int4(r, l, start_s[s] + j * beta, rows);
    }
    if (tid == 0) {
        int err = err_s;
        if (total > max_blocks) err |= 1;
        *n_blocks = total < max_blocks ? total : max_blocks;
        if (err_word) *err_word = err;
    }
}

}  // namespace

hipError_t moe_launch_plan(const int32_t* counts, int begin, int stride, int E_loc, int P,
                           int beta, int32_t* q, int32_t* moves, int32_t* n_moves,
                           int max_moves, int32_t* blocks, int32_t* n_blocks, int max_blocks,
                           int32_t* err_word, hipStream_t stream) {
    plan_kernel<<<1, kThreads, 0, stream>>>(counts, begin, stride, E_loc, P, beta, q, moves,
                                            n_moves, max_moves, blocks, n_blocks, max_blocks,
                                            err_word);
    return hipGetLastError();
}
