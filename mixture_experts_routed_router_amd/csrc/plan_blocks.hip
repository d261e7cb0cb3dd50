// plan_blocks.hip -- block-granular replica plan over logical rank partitions
// (moe_plan_blocks).
//
// MegaFlux §3.1 ("Problem formulation", "Bounded greedy search", "On-device planning and
// route construction") and App. A.1 ("Candidate construction", "Refinement"): each expert's
// rows are cut into blocks of at most beta rows; loads count blocks; four bounded greedy
// searches shift single blocks from ranks over tau = ceil(sum b / P) to replicas of their
// experts on ranks under tau, existing copies first, within a per-rank replica budget s; the
// smallest maximum load wins (then fewest replicas); replicas whose allocation fits
// elsewhere under that maximum are removed, then single blocks move from the busiest to the
// least busy rank where they share an expert.  The exact tie rules are stated in moe.h.
//
// One workgroup of four waves.  As on the pages, the four candidates run in parallel, one
// per wave: lane r holds rank r's load and replica count in registers, the candidate's
// block counts q[l][r] sit in LDS and lane r only touches column r of them (the donor's
// expert-scan snapshot excepted).  A donor's fan-out works on one expert row in registers
// (lane r = q[l][r]), so every single-block move is two wave reductions and a lane update.
// Every arg-min / arg-max is one branch-free reduction of 64-bit (value, index) keys over the
// whole wave (moe_wave.h), with the losing value in the lanes that do not compete.
// Selection, pruning (a bitonic sort of the replica keys by all threads, then wave 0) and
// the single-block pass follow; the table is emitted by all threads from per-(expert, rank)
// prefix sums, in the same layout as moe_plan's.
#include "moe_launch.h"
#include "moe_wave.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxCells = 4096;  // E_loc * P
constexpr int kBig = 0x7FFFFFFF;

// The cross-lane LDS traffic of a wave (the scan snapshot and the per-expert write-backs)
// goes through volatile accesses, which the compiler keeps in program order; a wave's LDS
// operations complete in issue order.
typedef volatile int vint;

// One greedy search; runs in one wave.  Returns through q (LDS) and the lane registers.
__device__ void search(vint* q, const int* b_s, int E_loc, int P, int G, int tau, int s,
                       bool by_overload, bool many, int lane, int& L, int& repl) {
    const bool rank_lane = lane < P;
    for (int i = lane; i < E_loc * P; i += MOE_WAVE) q[i] = 0;
    for (int l = lane; l < E_loc; l += MOE_WAVE) q[l * P + l / G] = b_s[l];
    L = 0;
    repl = 0;
    if (rank_lane)
        for (int l = lane * G; l < (lane + 1) * G; ++l) L += b_s[l];

    for (int64_t round = 0; round < (int64_t)s + 2; ++round) {
        bool moved = false;
        int key = -1;
        if (rank_lane && L > tau) {
            if (by_overload) {
                key = L - tau;
            } else {
                key = 0;
                for (int l = lane * G; l < (lane + 1) * G; ++l) key = max(key, (int)q[l * P + lane]);
            }
        }
        bool visited = false;
        for (;;) {
            int v = (!visited && key >= 0) ? key : -1, d = lane;
            wave_best_all<true>(v, d);
            if (v < 0) break;
            if (lane == d) visited = true;
            int Ld = __builtin_amdgcn_readlane(L, d);
            if (Ld <= tau) continue;
            // the donor's home experts with blocks at home, most blocks first (fixed at visit start)
            const int snap = lane < G ? (int)q[(d * G + lane) * P + d] : 0;
            bool scanned = false;
            while (Ld > tau) {
                int v2 = (lane < G && !scanned && snap > 0) ? snap : -1, j = lane;
                wave_best_all<true>(v2, j);
                if (v2 < 0) break;
                if (lane == j) scanned = true;
                const int l = d * G + j;
                int qc = rank_lane ? (int)q[l * P + lane] : 0;  // this lane's column of row l
                int qd = __builtin_amdgcn_readlane(qc, d);       // blocks of l still at home
                bool opened = false;                            // a new copy of l this round
                // Single-block moves, k at a time: the receiver stays the least-loaded eligible
                // copy (lower rank on ties) until it passes the runner-up, reaches tau, the
                // donor reaches tau or l runs out of blocks at home; a new copy is the only
                // eligible copy after its first block.  So k single-block steps in a row pick
                // the same receiver, and moving them at once gives the same plan.
                for (;;) {
                    if (qd == 0 || Ld <= tau) break;
                    const bool existing = rank_lane && lane != d && qc > 0 && L < tau;
                    int v3 = existing ? L : kBig, rcv = lane;
                    wave_best_all<false>(v3, rcv);
                    bool open_new = false;
                    int k = min(qd, Ld - tau);
                    if (v3 != kBig) {
                        int v5 = (existing && lane != rcv) ? L : kBig, r2 = lane;
                        wave_best_all<false>(v5, r2);
                        k = min(k, tau - v3);
                        if (v5 != kBig) k = min(k, rcv < r2 ? v5 - v3 + 1 : v5 - v3);
                    } else {
                        if (!many && opened) break;
                        int v4 = (rank_lane && lane != d && qc == 0 && repl < s && L < tau) ? L : kBig;
                        rcv = lane;
                        wave_best_all<false>(v4, rcv);
                        if (v4 == kBig) break;
                        open_new = true;
                        k = min(k, tau - v4);
                    }
                    if (lane == d) {
                        qc -= k;
                        L -= k;
                    }
                    if (lane == rcv) {
                        qc += k;
                        L += k;
                        if (open_new) repl += 1;
                    }
                    if (open_new) opened = true;
                    qd -= k;
                    Ld -= k;
                    moved = true;
                }
                if (rank_lane) q[l * P + lane] = qc;
            }
        }
        if (!moved) break;
    }
}

// Exclusive prefix of per-thread values over the workgroup in thread order; *total gets the
// sum.  part holds one int per wave.
__device__ __forceinline__ int block_scan(int v, int* part, int* total) {
    const int lane = moe_lane_id(), wave = threadIdx.x / MOE_WAVE;
    int incl = v;
#pragma unroll
    for (int d = 1; d < MOE_WAVE; d <<= 1) {
        const int o = __shfl_up(incl, d, MOE_WAVE);
        if (lane >= d) incl += o;
    }
    if (lane == MOE_WAVE - 1) part[wave] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kThreads / MOE_WAVE; ++w) {
        before += w < wave ? part[w] : 0;
        all += part[w];
    }
    *total = all;
    __syncthreads();  // part may be reused
    return before + incl - v;
}

__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, MOE_WAVE));
    return v;
}

__global__ void __launch_bounds__(kThreads)
plan_blocks_kernel(const int32_t* __restrict__ counts, int begin, int stride, int E_loc, int P,
                   int beta, int s, int32_t* __restrict__ q_out, int32_t* __restrict__ moves,
                   int32_t* __restrict__ n_moves, int max_moves, int32_t* __restrict__ blocks,
                   int32_t* __restrict__ n_blocks, int max_blocks,
                   int32_t* __restrict__ err_word) {
    __shared__ int n_s[256];
    __shared__ int b_s[256];
    __shared__ int off_s[257];
    __shared__ int qb[4][kMaxCells];            // candidates' block counts [l * P + r]
    __shared__ unsigned long long keys[kMaxCells];  // replica keys; then two prefix tables
    __shared__ int cand_max[4], cand_rep[4];
    __shared__ int part[kThreads / MOE_WAVE];
    __shared__ int sum_b_s, err_s;

    const int tid = threadIdx.x;
    const int lane = moe_lane_id();
    const int wave = tid / MOE_WAVE;
    const int G = E_loc / P;
    const int cells = E_loc * P;

    for (int l = tid; l < E_loc; l += kThreads) {
        const int n = counts[begin + l * stride];
        n_s[l] = n;
        b_s[l] = (n + beta - 1) / beta;
    }
    if (tid == 0) err_s = 0;
    __syncthreads();
    if (tid == 0) {
        int o = 0, sb = 0;
        for (int l = 0; l < E_loc; ++l) {
            off_s[l] = o;
            o += b_s[l] * beta;
            sb += b_s[l];
        }
        off_s[E_loc] = o;
        sum_b_s = sb;
    }
    __syncthreads();
    const int sum_b = sum_b_s;
    const int tau = (sum_b + P - 1) / P;

    // the four searches, one per wave: (overload, one copy), (overload, many),
    // (home load, one copy), (home load, many)
    {
        vint* q = qb[wave];
        int L, repl;
        search(q, b_s, E_loc, P, G, tau, s, wave < 2, (wave & 1) != 0, lane, L, repl);
        const int m = wave_max_i32(lane < P ? L : -1);
        int nr = 0;
        for (int i = lane; i < cells; i += MOE_WAVE) {
            const int l = i / P, r = i - l * P;
            nr += (r != l / G && q[i] > 0) ? 1 : 0;
        }
        nr = moe_wave_sum_i32(nr);
        if (lane == 0) {
            cand_max[wave] = m;
            cand_rep[wave] = nr;
        }
    }
    __syncthreads();
    int best = 0;
    for (int c = 1; c < 4; ++c)
        if (cand_max[c] < cand_max[best] ||
            (cand_max[c] == cand_max[best] && cand_rep[c] < cand_rep[best]))
            best = c;
    const int Lmax = cand_max[best];
    vint* q = qb[best];

    // pruning order: replicas by (allocation at pass entry, expert, rank); compacted by
    // wave 0, then sorted
    const int n_rep = cand_rep[best];
    int n2 = 1;
    while (n2 < n_rep) n2 <<= 1;
    if (wave == 0) {
        int base = 0;
        for (int c0 = 0; c0 < cells; c0 += MOE_WAVE) {
            const int c = c0 + lane;
            bool is_rep = false;
            unsigned long long k = 0;
            if (c < cells) {
                const int l = c / P, r = c - l * P;
                const int a = q[c];
                is_rep = r != l / G && a > 0;
                k = ((unsigned long long)a << 32) | ((unsigned long long)l << 16) | (unsigned)r;
            }
            const unsigned long long bal = __ballot(is_rep);
            if (is_rep) keys[base + __popcll(bal & ((1ull << lane) - 1))] = k;
            base += __popcll(bal);
        }
        for (int i = base + lane; i < n2; i += MOE_WAVE) keys[i] = ~0ull;
    }
    __syncthreads();
    for (int k = 2; k <= n2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < n2; i += kThreads) {
                const int p = i ^ j;
                if (p > i) {
                    const unsigned long long x = keys[i], y = keys[p];
                    const bool up = (i & k) == 0;
                    if (up ? x > y : x < y) {
                        keys[i] = y;
                        keys[p] = x;
                    }
                }
            }
            __syncthreads();
        }
    }

    if (wave == 0) {
        const bool rank_lane = lane < P;
        int L = 0;
        if (rank_lane)
            for (int l = 0; l < E_loc; ++l) L += q[l * P + lane];
        // refinement 1: drop replicas whose whole allocation fits under Lmax on the owner,
        // else on the least-loaded other copy
        for (int i = 0; i < n_rep; ++i) {
            const unsigned long long k = keys[i];
            const int l = (int)((k >> 16) & 0xFFFF), r = (int)(k & 0xFFFF), h = l / G;
            int qc = rank_lane ? (int)q[l * P + lane] : 0;
            const int a = __builtin_amdgcn_readlane(qc, r);
            if (a == 0) continue;
            int tgt = -1;
            if (__builtin_amdgcn_readlane(L, h) + a <= Lmax) {
                tgt = h;
            } else {
                int v = (rank_lane && lane != r && lane != h && qc > 0 && L + a <= Lmax) ? L : kBig;
                int t = lane;
                wave_best_all<false>(v, t);
                if (v != kBig) tgt = t;
            }
            if (tgt < 0) continue;
            if (lane == tgt) {
                qc += a;
                L += a;
            }
            if (lane == r) {
                qc = 0;
                L -= a;
            }
            if (rank_lane) q[l * P + lane] = qc;
        }
        // refinement 2: single blocks from the most- to the least-loaded rank
        for (int it = 0; it < sum_b; ++it) {
            int vmax = rank_lane ? L : -1, rmax = lane;
            wave_best_all<true>(vmax, rmax);
            int vmin = rank_lane ? L : kBig, rmin = lane;
            wave_best_all<false>(vmin, rmin);
            if (vmax - vmin <= 1) break;
            int lm = -1;
            for (int l0 = 0; l0 < E_loc && lm < 0; l0 += MOE_WAVE) {
                const int l = l0 + lane;
                const bool ok = l < E_loc && q[l * P + rmax] > 0 &&
                                (rmin == l / G || q[l * P + rmin] > 0);
                const unsigned long long bal = __ballot(ok);
                if (bal) lm = l0 + __ffsll((long long)bal) - 1;
            }
            if (lm < 0) break;
            if (lane == 0) {
                q[lm * P + rmax] = q[lm * P + rmax] - 1;
                q[lm * P + rmin] = q[lm * P + rmin] + 1;
            }
            if (lane == rmax) L -= 1;
            if (lane == rmin) L += 1;
        }
    }
    __syncthreads();

    // block table: expert l's blocks go to the ranks holding it in ascending rank order;
    // rows listed rank by rank, then expert by expert.  Two scans over the cells, 16
    // consecutive ones per thread: expert-major (each (l, r)'s first block within expert l,
    // rows per (l, r), the replica list in (expert, rank) order), then rank-major (each
    // (l, r)'s first position in the table); then one thread per table entry.
    constexpr int kPer = kMaxCells / kThreads;
    int* pre_l = reinterpret_cast<int*>(keys);  // first block of (l, r) within expert l
    const int c_lo = tid * kPer, c_hi = min(c_lo + kPer, cells);
    int my_blocks = 0, my_reps = 0;
    for (int c = c_lo; c < c_hi; ++c) {
        const int l = c / P, r = c - l * P, k = q[c];
        my_blocks += k;
        my_reps += (r != l / G && k > 0) ? 1 : 0;
    }
    int total_blocks, total_moves;
    int run_b = block_scan(my_blocks, part, &total_blocks);
    int run_m = block_scan(my_reps, part, &total_moves);
    for (int c = c_lo; c < c_hi; ++c) {
        const int l = c / P, r = c - l * P, k = q[c];
        const int pre = run_b - off_s[l] / beta;  // blocks of l on ranks below r
        pre_l[c] = pre;
        run_b += k;
        const int n = n_s[l];
        const int lo = min(n, pre * beta), hi = min(n, (pre + k) * beta);
        q_out[c] = hi - lo;
        if (r != l / G && k > 0) {
            if (run_m < max_moves) {
                int32_t* m = moves + 4 * run_m;
                m[0] = l / G;
                m[1] = r;
                m[2] = l;
                m[3] = hi - lo;
            } else {
                atomicOr(&err_s, 2);
            }
            ++run_m;
        }
    }
    __syncthreads();
    int my_rank_major = 0;
    for (int i = c_lo; i < c_hi; ++i) {
        const int r = i / E_loc, l = i - r * E_loc;
        my_rank_major += q[l * P + r];
    }
    int unused;
    int pos = block_scan(my_rank_major, part, &unused);
    int* start_rm = pre_l + kMaxCells;  // first table position of rank-major cell r * E_loc + l
    for (int i = c_lo; i < c_hi; ++i) {
        const int r = i / E_loc, l = i - r * E_loc;
        start_rm[i] = pos;
        pos += q[l * P + r];
    }
    __syncthreads();
    // one thread per table position: its cell is the last one starting at or before it
    // (cells without blocks share the next cell's start and are skipped that way)
    if (total_blocks > max_blocks && tid == 0) atomicOr(&err_s, 1);
    const int nb_out = min(total_blocks, max_blocks);
    for (int p = tid; p < nb_out; p += kThreads) {
        int lo = 0, hi = cells - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (start_rm[mid] <= p) lo = mid;
            else hi = mid - 1;
        }
        const int r = lo / E_loc, l = lo - r * E_loc;
        const int bi = pre_l[l * P + r] + (p - start_rm[lo]);
        int32_t* bl = blocks + 4 * p;
        bl[0] = r;
        bl[1] = l;
        bl[2] = off_s[l] + bi * beta;
        bl[3] = min(beta, n_s[l] - bi * beta);
    }
    __syncthreads();
    if (tid == 0) {
        *n_moves = min(total_moves, max_moves);
        *n_blocks = min(total_blocks, max_blocks);
        if (err_word) *err_word = err_s;
    }
}

}  // namespace

hipError_t moe_launch_plan_blocks(const int32_t* counts, int begin, int stride, int E_loc, int P,
                                  int beta, int s, int32_t* q, int32_t* moves, int32_t* n_moves,
                                  int max_moves, int32_t* blocks, int32_t* n_blocks,
                                  int max_blocks, int32_t* err_word, hipStream_t stream) {
    plan_blocks_kernel<<<1, kThreads, 0, stream>>>(counts, begin, stride, E_loc, P, beta, s, q,
                                                   moves, n_moves, max_moves, blocks, n_blocks,
                                                   max_blocks, err_word);
    return hipGetLastError();
}
