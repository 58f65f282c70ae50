// Persistent decode kernel: the whole drafter pass at low concurrency in one
// launch.
//
// [Blog] = "P-EAGLE: Faster LLM Inference with Parallel Speculative Decoding
// in vLLM" (summary page); [Paper] = "P-EAGLE: Parallel-Drafting EAGLE with
// Scalable Training" (summary page); [arXiv] = its ScienceStack page.
//
// At a few requests the drafter pass ([Blog] "P-EAGLE core method": every
// position goes through the layers and the LM head together) is a chain of
// weight streams (fc, then per layer QKV, O, gate/up, down, then the LM head)
// separated by small row-wise steps (norms, RoPE + KV write, attention). As
// separate kernels every link of the chain pays a launch and the ramp of a
// new weight stream. Here one cooperative launch of one workgroup per CU runs
// the chain as phases separated by grid barriers, and the weight stream never
// stops: the LDS ring that feeds the matrix cores keeps loading the next
// projection's weights (which depend on nothing) while the workgroup waits at
// a barrier or works on a row phase, and only the activation columns of a
// stage wait for the barrier that makes them ready.
//
// Phases of one pass (N layers):
//   fc GEMM (split-K planes) | layer-0 input + attention plan |
//   per layer: QKV GEMM | RoPE + KV write | attention splits | merge |
//              O GEMM | residual + RMSNorm | gate/up GEMM (SwiGLU) | down GEMM |
//              residual + RMSNorm (the last layer: final norm of the sampled rows) |
//   LM head GEMM with per-wave argmax partials | argmax of every sampled row.
// Data handed from one phase to the next goes through memory with coherent
// (sc1) stores and loads (common.hpp ldc / stc): the XCDs' L2 caches are not
// coherent with one another, and flushing them at every barrier measured
// slower than writing through.
#include <float.h>
#include <limits.h>

#include <cstring>

#include "attn_dev.hpp"

namespace pd {

namespace {

constexpr int kNT = 256;          // threads per workgroup (4 waves)
constexpr int kRS = 128;          // reduction elements per ring stage
constexpr int kWR = 64;           // weight rows per stage: 16 per wave
constexpr int kAttnStages = 2;    // attention page ring depth inside the decode kernel
constexpr int kPlanMaxC = 64;     // requests the decode kernel accepts
constexpr unsigned kSpinLimit = 1u << 22;   // barrier polls before a wait gives up

__device__ __align__(16) uint16_t g_dec_zero[8];

// Ring geometry per 16-row X tile count MT: stage = 64 weight rows + 16 MT
// activation rows of kRS elements; as many stages as the LDS left by the
// attention region holds.
template <int MT>
struct DecRing {
    static constexpr int XR = 16 * MT;
    static constexpr int WL = kWR * 16 / kNT;   // 16-byte weight copies per thread per stage (4)
    static constexpr int XL = XR * 16 / kNT;    // activation copies per thread per stage (MT)
    static constexpr int L = WL + XL;
    static constexpr int SE = (kWR + XR) * kRS; // elements per stage
    static constexpr int NST = MT == 1 ? 6 : (MT == 2 ? 5 : 3);
};

__device__ __forceinline__ unsigned lds_off(void* p) {
    return __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)p);
}

template <int N>
__device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
template <int L, int MAXN>
__device__ __forceinline__ void vm_wait_later(int later) {
    if constexpr (MAXN == 0) {
        vm_wait<0>();
    } else {
        if (later >= MAXN) vm_wait<L * MAXN>();
        else vm_wait_later<L, MAXN - 1>(later);
    }
}
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ void better_f(float& bv, int& bi, float ov, int oi) {
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
}

__device__ __forceinline__ uint2 pack4_bf(float a, float b, float c, float d) {
    uint2 pk;
    pk.x = uint32_t(f2bf(a)) | (uint32_t(f2bf(b)) << 16);
    pk.y = uint32_t(f2bf(c)) | (uint32_t(f2bf(d)) << 16);
    return pk;
}

}  // namespace

namespace {

// ------------------------------------------------------------------ barrier
// Generation barrier over the grid: each workgroup writes its arrival word,
// the last workgroup waits for all of them and writes the release word, the
// others wait for that. Generations continue from the release word's value at the
// start of the launch, so nothing has to be reset between launches. Every
// wait gives up after kSpinLimit polls (status PD_STATUS_SYNC_TIMEOUT): no
// wave can wait forever.
struct GridBar {
    unsigned* w;
    unsigned gen;
    bool alive;
};

__device__ __forceinline__ unsigned ld_sync(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sync(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// later: weight copies (in units of L per ring stage) this workgroup issued
// after its last store of the phase; they stay in flight
template <int L, int MAXN>
__device__ __forceinline__ void grid_barrier(GridBar& b, int32_t* status, uint64_t* tl, int later) {
    __shared__ int s_ok;
    const unsigned G = gridDim.x;
    const unsigned M = G - 1;   // the master: a row workgroup, which never streams weights ahead
    const unsigned gen = ++b.gen;
    // every wave's stores of the phase (written through) are done; the
    // counter is per wave and in order, and the weight copies issued after
    // the stores may stay in flight
    vm_wait_later<L, MAXN>(later);
    __syncthreads();
    if (threadIdx.x == 0) {
        if (tl) tl[blockIdx.x] = __builtin_amdgcn_s_memrealtime();
        st_sync(b.w + 64 + blockIdx.x, gen);
    }
    if (blockIdx.x == M) {
        bool done = !b.alive;
        for (unsigned spins = 0; !done; ++spins) {
            const bool mine = threadIdx.x >= G || (int)(ld_sync(b.w + 64 + threadIdx.x) - gen) >= 0;
            done = __syncthreads_and(mine);
            if (!done && spins >= kSpinLimit) {
                if (threadIdx.x == 0) flag(status, PD_STATUS_SYNC_TIMEOUT);
                b.alive = false;
                break;
            }
        }
        if (threadIdx.x == 0 && b.alive) st_sync(b.w, gen);
    }
    if (threadIdx.x == 0) {
        int ok = b.alive;
        if (ok && blockIdx.x != M) {
            for (unsigned spins = 0; (int)(ld_sync(b.w) - gen) < 0; ++spins) {
                if (spins >= kSpinLimit) {
                    flag(status, PD_STATUS_SYNC_TIMEOUT);
                    ok = 0;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        s_ok = ok;
    }
    __syncthreads();
    b.alive = s_ok;
}

// ------------------------------------------------------------------ GEMM jobs
// Per-layer weight pointers and per-kind projection parameters, copied from
// the kernel arguments to LDS once: selecting argument fields by a run-time
// layer or projection kind would make the compiler copy the whole argument
// block to scratch memory. Values read back are made wave-uniform.
enum LayerPtr { LP_QKV, LP_O, LP_GATE, LP_UP, LP_DOWN, LP_NORM_IN, LP_NORM_POST, LP_COUNT };
enum JobKind { JK_FC, JK_QKV0, JK_QKV, JK_O, JK_GU, JK_DOWN, JK_LM, JK_COUNT };
struct JobParams {
    const uint16_t* X;
    int ldx, M, N, K, splits, grid, epi;
};
struct Tables {
    const uint16_t* lp[LP_COUNT][PD_MAX_LAYERS];
    JobParams jk[JK_COUNT];
    size_t u_slot, ao_slot, act_slot;
    uint16_t* act;
};

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename T>
__device__ __forceinline__ T* uni_ptr(T* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<T*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ void load_tables(const DecodeArgs& a, Tables& t) {
    if (threadIdx.x != 0) return;
#pragma unroll
    for (int l = 0; l < PD_MAX_LAYERS; ++l) {
        t.lp[LP_QKV][l] = a.w_qkv[l];
        t.lp[LP_O][l] = a.w_o[l];
        t.lp[LP_GATE][l] = a.w_gate[l];
        t.lp[LP_UP][l] = a.w_up[l];
        t.lp[LP_DOWN][l] = a.w_down[l];
        t.lp[LP_NORM_IN][l] = a.norm_in[l];
        t.lp[LP_NORM_POST][l] = a.norm_post[l];
    }
    const int qkvw = (a.Hq + 2 * a.Hkv) * a.dh, hd = a.Hq * a.dh;
    t.jk[JK_FC] = JobParams{a.hidden, a.hidden3, a.T, a.d, a.hidden3, a.sp_fc, a.hidden_d ? 0 : a.g_fc, EPI_PARTIAL};
    t.jk[JK_QKV0] = JobParams{a.u, 2 * a.d, a.T, qkvw, 2 * a.d, a.sp_qkv0, a.g_qkv0, EPI_PARTIAL};
    t.jk[JK_QKV] = JobParams{a.u, a.d, a.T, qkvw, a.d, a.sp_qkv, a.g_qkv, EPI_PARTIAL};
    t.jk[JK_O] = JobParams{a.ao, hd, a.T, a.d, hd, a.sp_o, a.g_o, EPI_PARTIAL};
    t.jk[JK_GU] = JobParams{a.u, a.d, a.T, a.F, a.d, 1, a.g_gu, EPI_SWIGLU};
    t.jk[JK_DOWN] = JobParams{a.act, a.F, a.T, a.d, a.F, a.sp_down, a.g_down, EPI_PARTIAL};
    t.jk[JK_LM] = JobParams{a.xg, a.d, a.R, a.V, a.d, 1, a.lm_in_kernel ? a.g_lm : 0, EPI_ARGMAX};
    t.u_slot = a.u_slot;
    t.ao_slot = a.ao_slot;
    t.act_slot = a.act_slot;
    t.act = a.act;
}

// Job j of the pass: 0 = fc, 1 + 4l + {0 QKV, 1 O, 2 gate/up, 3 down}, 1 + 4N = LM head.
struct Job {
    const uint16_t* W;
    const uint16_t* W2;    // up matrix (SwiGLU pair), else null
    const uint16_t* X;     // bf16 activation rows
    uint16_t* Y;           // SwiGLU output rows
    int ldx, M, N, K, splits, grid, epi;
};

__device__ __forceinline__ int job_kind(int j, int nj) {
    if (j <= 0) return JK_FC;
    if (j >= nj - 1) return JK_LM;
    const int l = (j - 1) >> 2, k = (j - 1) & 3;
    return k == 0 ? (l == 0 ? JK_QKV0 : JK_QKV) : (k == 1 ? JK_O : (k == 2 ? JK_GU : JK_DOWN));
}

__device__ __forceinline__ Job make_job(const Tables& t, const DecodeArgs& a, int j, int nj) {
    Job b;
    const int kind = job_kind(j, nj);
    const JobParams& jp = t.jk[kind];
    b.X = uni_ptr(jp.X);
    b.ldx = uni(jp.ldx); b.M = uni(jp.M); b.N = uni(jp.N); b.K = uni(jp.K);
    b.splits = uni(jp.splits); b.grid = uni(jp.grid); b.epi = uni(jp.epi);
    b.W2 = nullptr;
    b.Y = nullptr;
    const int l = j >= 1 ? (j - 1) >> 2 : 0;
    // the activation slot this projection reads
    if (kind == JK_QKV) b.X += (size_t)(2 * l) * t.u_slot;
    else if (kind == JK_GU) b.X += (size_t)(2 * l + 1) * t.u_slot;
    else if (kind == JK_O) b.X += (size_t)l * t.ao_slot;
    else if (kind == JK_DOWN) b.X += (size_t)l * t.act_slot;
    if (kind == JK_GU) b.Y = uni_ptr(t.act) + (size_t)l * t.act_slot;
    if (kind == JK_FC) b.W = a.fc;
    else if (kind == JK_LM) b.W = a.lm_head;
    else {
        const int lp = (kind == JK_QKV0 || kind == JK_QKV) ? LP_QKV : (kind == JK_O ? LP_O : (kind == JK_GU ? LP_GATE : LP_DOWN));
        b.W = uni_ptr(t.lp[lp][l]);
        if (kind == JK_GU) b.W2 = uni_ptr(t.lp[LP_UP][l]);
    }
    if (j >= nj || j < 0) b.grid = 0;
    return b;
}

// columns per item: 64 (16 per wave), or 32 for the gate/up pair (waves 0, 1
// gate rows, waves 2, 3 the same columns' up rows)
__device__ __forceinline__ int job_tw(const Job& b) { return b.epi == EPI_SWIGLU ? 32 : 64; }

// The weight ring of one workgroup. The issue cursor walks (job, item, stage)
// in the order the consumer will; it may run ahead into the next job while
// that job's activations are not ready yet: such stages get their weights
// now and zeros (the 16 zero bytes) in their activation slots, and the real
// activation copies are issued once the job's phase begins. Every stage
// therefore carries exactly WL + XL copies per thread, which keeps the
// in-order vmcnt accounting of the waits.
template <int MT>
struct RingEngine {
    using Cf = DecRing<MT>;
    static constexpr int NST = Cf::NST, WL = Cf::WL, XL = Cf::XL, L = Cf::L;

    uint16_t* ring;      // LDS
    const Tables* tb;     // LDS
    unsigned lds0;
    int nj;              // jobs in the pass
    // issue cursor
    int ij, iit, iks, ike;   // job, item, stage, item's stage end
    Job ib;                  // job ij
    int ready_job;           // activations of jobs <= ready_job may be copied
    int pre_job, npre;       // stages issued with zero activations: all of job pre_job
    int issued;              // stages issued so far
    const uint16_t* wp[WL];
    bool wfull;
    const uint16_t* xp[XL];
    int xch[XL];
    int wofs[WL], wrr[WL];

    __device__ __forceinline__ void init(uint16_t* r, int njobs) {
        ring = r;
        lds0 = lds_off(r);
        nj = njobs;
        ready_job = -1;
        pre_job = -1;
        npre = 0;
        issued = 0;
        ahead = false;
        const int tid = threadIdx.x;
#pragma unroll
        for (int j = 0; j < WL; ++j) {
            const int u = tid + kNT * j, wr = u >> 4;
            wrr[j] = wr;
            wofs[j] = ((u & 15) ^ (wr & 15)) * 8;
        }
#pragma unroll
        for (int j = 0; j < XL; ++j) {
            const int u = tid + kNT * j, m = u >> 4;
            xch[j] = ((u & 15) ^ (m & 15)) * 8;
        }
    }

    __device__ __forceinline__ static int ksteps(const Job& b) { return (b.K + kRS - 1) / kRS; }
    __device__ __forceinline__ static int per(const Job& b) { return (ksteps(b) + b.splits - 1) / b.splits; }
    __device__ __forceinline__ static int ntn(const Job& b) { return (b.N + job_tw(b) - 1) / job_tw(b); }
    __device__ __forceinline__ static int nitems(const Job& b) { return ntn(b) * b.splits; }

    // weight sources of item it of job b, and the item's stage range
    __device__ __forceinline__ void set_item(const Job& b, int it) {
        const int sp = it / ntn(b);
        iks = sp * per(b);
        ike = min(ksteps(b), (sp + 1) * per(b));
        const int tw = job_tw(b);
        const int n0 = (it % ntn(b)) * tw;
        wfull = n0 + tw <= b.N;
#pragma unroll
        for (int j = 0; j < WL; ++j) {
            int row = wrr[j];
            const uint16_t* base = b.W;
            if (b.W2 && row >= 32) { base = b.W2; row -= 32; }
            const int n = n0 + row;
            wp[j] = n < b.N ? base + (size_t)n * b.K + wofs[j] : nullptr;
        }
    }
    __device__ __forceinline__ void set_x(const Job& b) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int j = 0; j < XL; ++j) {
            const int m = (tid + kNT * j) >> 4;
            xp[j] = m < b.M ? b.X + (size_t)m * b.ldx : nullptr;
        }
    }
    // move the cursor to the next (job, item) with stages, starting at job j, item it
    __device__ __forceinline__ void seek(const DecodeArgs& a, int j, int it) {
        ij = j;
        while (ij < nj) {
            ib = make_job(*tb, a, ij, nj);
            if (blockIdx.x < (unsigned)ib.grid) {
                const int n = nitems(ib);
                for (iit = it; iit < n; iit += ib.grid) {
                    set_item(ib, iit);
                    if (iks < ike) {
                        set_x(ib);
                        return;
                    }
                }
            }
            ++ij;
            it = blockIdx.x;
        }
    }
    __device__ __forceinline__ void start(const DecodeArgs& a, uint16_t* r, const Tables* table) {
        tb = table;
        init(r, 2 + 4 * a.NL);
        seek(a, 0, blockIdx.x);
    }

    // may the cursor issue its current stage now? Stages of a job whose
    // activations are not ready only at a prefetch point (ahead), and all of
    // one job
    bool ahead;
    __device__ __forceinline__ bool can_issue() const {
        if (ij >= nj) return false;
        if (ij <= ready_job) return true;
        return ahead && (npre == 0 || pre_job == ij);
    }
    // Weights of the next job's first stages, into the free slots (after the
    // phase's stores: the barrier then waits only for those). qc: stages
    // consumed. Returns the stages issued.
    __device__ __forceinline__ int prefetch(const DecodeArgs& a, int qc) {
        ahead = true;
        int n = 0;
        while (issued - qc < NST - 1 && can_issue()) {
            issue(a);
            ++n;
        }
        ahead = false;
        return n;
    }

    // issue the cursor's stage into its slot and advance the cursor
    __device__ __forceinline__ void issue(const DecodeArgs& a) {
        const int slot = issued % NST;
        const unsigned sbase = lds0 + (unsigned)(slot * Cf::SE) * 2u;
        const int wave = threadIdx.x >> 6;
        const int k0 = iks * kRS;
        const bool kin = k0 + kRS <= ib.K;
        const bool inner = wfull && kin;
        const uint16_t* zp = g_dec_zero;
#pragma unroll
        for (int j = 0; j < WL; ++j) {
            const uint16_t* src;
            if (inner) src = wp[j] + k0;
            else src = (wp[j] && k0 + wofs[j] < ib.K) ? wp[j] + k0 : zp;
            __builtin_amdgcn_global_load_lds((void*)src,
                (__attribute__((address_space(3))) void*)(uintptr_t)(sbase + (unsigned)(wave * 64 + kNT * j) * 16u),
                16, 0, 2);   // weights are read once: non-temporal
        }
        const bool real = ij <= ready_job;
#pragma unroll
        for (int j = 0; j < XL; ++j) {
            const int k = k0 + xch[j];
            const uint16_t* src = (real && xp[j] && (kin || k < ib.K)) ? xp[j] + k : zp;
            __builtin_amdgcn_global_load_lds((void*)src,
                (__attribute__((address_space(3))) void*)(uintptr_t)(sbase + (unsigned)(kWR * kRS * 2) +
                                                                      (unsigned)(wave * 64 + kNT * j) * 16u),
                16, 0, 0);   // write-once slots: no stale copy in any L2
        }
        if (!real) {
            pre_job = ij;
            ++npre;
        }
        ++issued;
        if (++iks >= ike) seek(a, ij, iit + ib.grid);
    }

    // real activation copies for the npre stages of job j issued ahead with
    // zeros (the first npre stages of this workgroup in job j, in order),
    // into slots first_slot, first_slot + 1, ...
    __device__ __forceinline__ void fill_pre(const Job& b, int first_stage) {
        set_x(b);
        const int wave = threadIdx.x >> 6;
        const uint16_t* zp = g_dec_zero;
        int it = blockIdx.x, ks = 0, ke = 0;
        auto item_range = [&](int item) {
            const int sp = item / ntn(b);
            ks = sp * per(b);
            ke = min(ksteps(b), (sp + 1) * per(b));
        };
        const int n = nitems(b);
        item_range(it);
        while (ks >= ke && it < n) { it += b.grid; if (it < n) item_range(it); }
        for (int i = 0; i < npre; ++i) {
            const int slot = (first_stage + i) % NST;
            const unsigned sbase = lds0 + (unsigned)(slot * Cf::SE) * 2u;
            const int k0 = ks * kRS;
            const bool kin = k0 + kRS <= b.K;
#pragma unroll
            for (int j = 0; j < XL; ++j) {
                const int k = k0 + xch[j];
                const uint16_t* src = (xp[j] && (kin || k < b.K)) ? xp[j] + k : zp;
                __builtin_amdgcn_global_load_lds((void*)src,
                    (__attribute__((address_space(3))) void*)(uintptr_t)(sbase + (unsigned)(kWR * kRS * 2) +
                                                                          (unsigned)(wave * 64 + kNT * j) * 16u),
                    16, 0, 0);
            }
            if (++ks >= ke) {
                do { it += b.grid; if (it < n) item_range(it); } while (it < n && ks >= ke);
            }
        }
        npre = 0;
        pre_job = -1;
    }
};

// ------------------------------------------------------------------ GEMM phase
// Consume this workgroup's stages of job j (all of its items), issuing ahead.
// qc: stages consumed so far (the ring slot of stage qc is qc % NST).
template <int MT>
__device__ __forceinline__ void gemm_phase(const DecodeArgs& a, RingEngine<MT>& R, int j, int& qc, float* xchg) {
    using Cf = DecRing<MT>;
    constexpr int NST = Cf::NST, L = Cf::L;
    const Job b = make_job(*R.tb, a, j, R.nj);
    R.ready_job = j;
    // activations of the stages issued ahead with zeros (they are all of job j
    // when this workgroup has stages in job j)
    if (R.npre > 0 && R.pre_job == j) R.fill_pre(b, qc);
    // fill the ring
    while (R.issued - qc < NST - 1 && R.can_issue()) R.issue(a);
    vm_wait<0>();
    if (blockIdx.x >= (unsigned)b.grid) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g4 = lane >> 4;
    const int ntn = RingEngine<MT>::ntn(b), nit = RingEngine<MT>::nitems(b);
    const int ks_all = RingEngine<MT>::ksteps(b), per = RingEngine<MT>::per(b);
    const int tw = job_tw(b);
    float runv[MT];
    int runi[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        runv[t] = -FLT_MAX;
        runi[t] = INT_MAX;
    }
    for (int it = blockIdx.x; it < nit; it += b.grid) {
        const int sp = it / ntn;
        const int kb = sp * per, ke = min(ks_all, (sp + 1) * per);
        if (kb >= ke) continue;
        f32x4 acc[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int ks = kb; ks < ke; ++ks, ++qc) {
            vm_wait_later<L, NST - 2>(min(NST - 2, R.issued - 1 - qc));
            lds_barrier();
            if (R.issued - qc < NST && R.can_issue()) R.issue(a);
            const uint16_t* Ws = R.ring + (qc % NST) * Cf::SE;
            const uint16_t* Xs = Ws + kWR * kRS;
#pragma unroll
            for (int jj = 0; jj < kRS / 32; ++jj) {
                const int pos = ((4 * jj + g4) ^ r16) * 8;
                const bf16x8 wf = *reinterpret_cast<const bf16x8*>(Ws + (16 * wave + r16) * kRS + pos);
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const bf16x8 xf = *reinterpret_cast<const bf16x8*>(Xs + (16 * t + r16) * kRS + pos);
                    acc[t] = mfma_16x16x32(wf, xf, acc[t]);
                }
            }
        }
        // lane holds columns n .. n+3 of rows m = 16t + r16
        const int n0 = (it % ntn) * tw;
        if (b.epi == EPI_PARTIAL) {
            const int n = n0 + 16 * wave + 4 * g4;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int m = 16 * t + r16;
                if (m < b.M && n < b.N)
                    stc<true>(reinterpret_cast<f32x4*>(a.ws + ((size_t)sp * b.M + m) * b.N + n), acc[t]);
            }
        } else if (b.epi == EPI_SWIGLU) {
            // waves 2, 3 hand their up columns to waves 0, 1 through LDS
            __syncthreads();
            if (wave >= 2) {
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    *reinterpret_cast<f32x4*>(xchg + ((t * 2 + (wave - 2)) * 64 + lane) * 4) = acc[t];
            }
            __syncthreads();
            if (wave < 2) {
                const int n = n0 + 16 * wave + 4 * g4;
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const int m = 16 * t + r16;
                    const f32x4 up = *reinterpret_cast<const f32x4*>(xchg + ((t * 2 + wave) * 64 + lane) * 4);
                    if (m < b.M && n < b.N)
                        stc<true>(reinterpret_cast<uint2*>(b.Y + (size_t)m * a.F + n),
                                  pack4_bf(silu_f(acc[t][0]) * up[0], silu_f(acc[t][1]) * up[1],
                                           silu_f(acc[t][2]) * up[2], silu_f(acc[t][3]) * up[3]));
                }
            }
        } else {   // EPI_ARGMAX
            const int n = n0 + 16 * wave + 4 * g4;
            if (n < b.N) {
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const int m = 16 * t + r16;
#pragma unroll
                    for (int e = 0; e < 4; ++e) better_f(runv[t], runi[t], acc[t][e], n + e);
                    if (a.logits && m < b.M)
                        *reinterpret_cast<f32x4*>(a.logits + (size_t)m * b.N + n) = acc[t];
                }
            }
        }
    }
    if (b.epi == EPI_ARGMAX) {
        const int ntiles = b.grid * 4;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            float bv = runv[t];
            int bi = runi[t];
#pragma unroll
            for (int off = 16; off <= 32; off <<= 1) {
                const float ov = __shfl_xor(bv, off, kWave);
                const int oi = __shfl_xor(bi, off, kWave);
                better_f(bv, bi, ov, oi);
            }
            const int m = 16 * t + r16;
            if (g4 == 0 && m < b.M) {
                stc<true>(a.amax_v + (size_t)m * ntiles + blockIdx.x * 4 + wave, bv);
                stc<true>(a.amax_i + (size_t)m * ntiles + blockIdx.x * 4 + wave, bi);
            }
        }
    }
}

// ------------------------------------------------------------------ row phases
constexpr int kRowNC = 4;   // 4 floats per thread per chunk, d <= 4096

__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

// sum of a projection's S split planes for row o, columns c .. c+3
__device__ __forceinline__ float4 planes_sum(const float* ws, int S, int T, int N, int o, int c) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 p[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
        if (s < S) p[s] = ldc<true>(reinterpret_cast<const float4*>(ws + ((size_t)s * T + o) * N + c));
#pragma unroll
    for (int s = 0; s < 8; ++s)
        if (s < S) { v.x += p[s].x; v.y += p[s].y; v.z += p[s].z; v.w += p[s].w; }
    return v;
}

// layer-0 input of row o ([Blog] Input_i equation): x = fc(h) (or the given
// d-wide row), u = [RMSNorm(E[id]; g_emb) || RMSNorm(x; g_hid)]
__device__ __forceinline__ void layer0_row(const DecodeArgs& a, int o, int S, float* red) {
    const int d = a.d;
    int id = a.ids[o];
    if (id < 0 || id >= a.V) {
        if (threadIdx.x == 0) flag(a.status, PD_STATUS_BAD_TOKEN);
        id = 0;
    }
    const uint16_t* er = a.embed + (size_t)id * d;
    float4 v[kRowNC];
    float ev[kRowNC][4];
    float se = 0.f, sx = 0.f;
#pragma unroll
    for (int n = 0; n < kRowNC; ++n) {
        const int c = threadIdx.x * 4 + 1024 * n;
        v[n] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (c < d) {
            if (a.hidden_d) {
                const uint2 hb = *reinterpret_cast<const uint2*>(a.hidden_d + (size_t)o * d + c);
                v[n] = make_float4(bf2f(hb.x & 0xffff), bf2f(hb.x >> 16), bf2f(hb.y & 0xffff), bf2f(hb.y >> 16));
            } else {
                v[n] = planes_sum(a.ws, S, a.T, d, o, c);
            }
            const uint2 eb = *reinterpret_cast<const uint2*>(er + c);
            ev[n][0] = bf2f(eb.x & 0xffff); ev[n][1] = bf2f(eb.x >> 16);
            ev[n][2] = bf2f(eb.y & 0xffff); ev[n][3] = bf2f(eb.y >> 16);
            stc<true>(reinterpret_cast<float4*>(a.x + (size_t)o * d + c), v[n]);
            if (a.dbg) *reinterpret_cast<float4*>(a.dbg + (size_t)o * d + c) = v[n];
            se += ev[n][0] * ev[n][0] + ev[n][1] * ev[n][1] + ev[n][2] * ev[n][2] + ev[n][3] * ev[n][3];
            sx += v[n].x * v[n].x + v[n].y * v[n].y + v[n].z * v[n].z + v[n].w * v[n].w;
        }
    }
    se = block_sum(se, red);
    sx = block_sum(sx, red);
    const float re = 1.0f / sqrtf(se / (float)d + a.eps);
    const float rx = 1.0f / sqrtf(sx / (float)d + a.eps);
    uint16_t* ur = a.u + (size_t)o * 2 * d;
#pragma unroll
    for (int n = 0; n < kRowNC; ++n) {
        const int c = threadIdx.x * 4 + 1024 * n;
        if (c < d) {
            const uint2 ge = *reinterpret_cast<const uint2*>(a.norm_emb + c);
            const uint2 gh = *reinterpret_cast<const uint2*>(a.norm_hid + c);
            stc<true>(reinterpret_cast<uint2*>(ur + c),
                      pack4_bf(ev[n][0] * re * bf2f(ge.x & 0xffff), ev[n][1] * re * bf2f(ge.x >> 16),
                               ev[n][2] * re * bf2f(ge.y & 0xffff), ev[n][3] * re * bf2f(ge.y >> 16)));
            stc<true>(reinterpret_cast<uint2*>(ur + d + c),
                      pack4_bf(v[n].x * rx * bf2f(gh.x & 0xffff), v[n].y * rx * bf2f(gh.x >> 16),
                               v[n].z * rx * bf2f(gh.y & 0xffff), v[n].w * rx * bf2f(gh.y >> 16)));
        }
    }
}

// residual update of row i (x += the projection's planes) and its RMSNorm:
// out row o = bf16(gamma * x / rms). write_x: store the updated row back.
__device__ __forceinline__ void resid_norm_row(const DecodeArgs& a, int i, int o, int S, const uint16_t* gamma, uint16_t* out,
                               bool write_x, float* snap, uint16_t* xout, float* red) {
    const int d = a.d;
    float4 v[kRowNC];
    float ss = 0.f;
#pragma unroll
    for (int n = 0; n < kRowNC; ++n) {
        const int c = threadIdx.x * 4 + 1024 * n;
        v[n] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (c < d) {
            const float4 xv = ldc<true>(reinterpret_cast<const float4*>(a.x + (size_t)i * d + c));
            const float4 pv = planes_sum(a.ws, S, a.T, d, i, c);
            v[n] = make_float4(xv.x + pv.x, xv.y + pv.y, xv.z + pv.z, xv.w + pv.w);
            if (write_x) stc<true>(reinterpret_cast<float4*>(a.x + (size_t)i * d + c), v[n]);
            if (snap) *reinterpret_cast<float4*>(snap + (size_t)i * d + c) = v[n];
            if (xout) *reinterpret_cast<uint2*>(xout + (size_t)o * d + c) = pack4_bf(v[n].x, v[n].y, v[n].z, v[n].w);
            ss += v[n].x * v[n].x + v[n].y * v[n].y + v[n].z * v[n].z + v[n].w * v[n].w;
        }
    }
    ss = block_sum(ss, red);
    const float rs = 1.0f / sqrtf(ss / (float)d + a.eps);
    if (!out) return;
#pragma unroll
    for (int n = 0; n < kRowNC; ++n) {
        const int c = threadIdx.x * 4 + 1024 * n;
        if (c < d) {
            const uint2 gb = *reinterpret_cast<const uint2*>(gamma + c);
            stc<true>(reinterpret_cast<uint2*>(out + (size_t)o * d + c),
                      pack4_bf(v[n].x * rs * bf2f(gb.x & 0xffff), v[n].y * rs * bf2f(gb.x >> 16),
                               v[n].z * rs * bf2f(gb.y & 0xffff), v[n].w * rs * bf2f(gb.y >> 16)));
        }
    }
}

// RoPE of q and k at each row's position and the paged K/V write
// ([Blog] KV-cache paragraph: slot -1 writes nothing), one thread per rotation
// pair or V element, spread over the grid; the angle is formed and reduced in
// double precision as in the row kernel of the same step.
__device__ __forceinline__ void rope_phase(const DecodeArgs& a, int S, uint16_t* kpl, uint16_t* vpl) {
    const int dh = a.dh, half = dh / 2;
    const int npairs = (a.Hq + a.Hkv) * half;
    const int per_row = npairs + a.Hkv * dh;
    const int W = (a.Hq + 2 * a.Hkv) * dh;
    const int total = a.T * per_row;
    for (int g = blockIdx.x * kNT + threadIdx.x; g < total; g += gridDim.x * kNT) {
        const int o = g / per_row, item = g % per_row;
        const int slot = a.slots[o];
        const bool write = slot >= 0 && slot < a.num_blocks * PD_PAGE;
        if (slot >= a.num_blocks * PD_PAGE && item == 0) flag(a.status, PD_STATUS_BAD_PAGE);
        const int blk = slot / PD_PAGE, off = slot % PD_PAGE;
        if (item < npairs) {
            const int h = item / half, i = item % half;
            const int c0 = h * dh + i;
            float pa[8], pb[8];
#pragma unroll
            for (int s = 0; s < 8; ++s)
                if (s < S) {
                    pa[s] = ldc<true>(a.ws + ((size_t)s * a.T + o) * W + c0);
                    pb[s] = ldc<true>(a.ws + ((size_t)s * a.T + o) * W + c0 + half);
                }
            float x0a = 0.f, x1a = 0.f;
#pragma unroll
            for (int s = 0; s < 8; ++s)
                if (s < S) { x0a += pa[s]; x1a += pb[s]; }
            const int pos = a.positions[o];
            double inv = 1.0, pw = a.inv_step;
            for (int e = i; e != 0; e >>= 1) {
                if (e & 1) inv *= pw;
                pw *= pw;
            }
            const double ang = (double)pos * inv;
            const double kq = rint(ang * 0.15915494309189535);
            double red = fma(-kq, 6.283185307179586, ang);
            red = fma(-kq, 2.4492935982947064e-16, red);
            float sn, cs;
            sincosf((float)red, &sn, &cs);
            const float x0 = x0a * cs - x1a * sn, x1 = x1a * cs + x0a * sn;
            if (h < a.Hq) {
                stc<true>(a.q + (size_t)o * a.Hq * dh + c0, f2bf(x0));
                stc<true>(a.q + (size_t)o * a.Hq * dh + c0 + half, f2bf(x1));
            } else if (write) {
                uint16_t* kp = kpl + ((size_t)blk * a.Hkv + (h - a.Hq)) * PD_PAGE * dh + off * dh;
                stc<true>(kp + i, f2bf(x0));
                stc<true>(kp + i + half, f2bf(x1));
            }
        } else if (write) {
            const int idx = item - npairs;
            float pv[8], v = 0.f;
#pragma unroll
            for (int s = 0; s < 8; ++s)
                if (s < S) pv[s] = ldc<true>(a.ws + ((size_t)s * a.T + o) * W + (a.Hq + a.Hkv) * dh + idx);
#pragma unroll
            for (int s = 0; s < 8; ++s)
                if (s < S) v += pv[s];
            const int gh = idx / dh, cc = idx % dh;
            stc<true>(vpl + ((size_t)blk * a.Hkv + gh) * PD_PAGE * dh + cc * PD_PAGE + off, f2bf(v));
        }
    }
}

// LDS shared by phases that never overlap: the attention page ring, the
// gate/up exchange and the norms' reductions
template <int DH>
union PhaseSmem {
    AttnSmem<DH, false, kAttnStages> at;
    float xchg[4 * 2 * 64 * 4];
    float red[8];
};

// ------------------------------------------------------------------ the kernel
// Workgroups 0 .. rows0 - 1 stream the projections (and stream the next
// projection's first weight stages ahead, after their own stores of a
// phase); workgroups rows0 .. G - 1, one per row, do the row phases and never
// stream ahead, so that their loads never queue behind weight copies (the
// vector-memory counter is per wave and in order). Everyone takes part in
// RoPE, attention and the merge, after which no weights are in flight.
template <int MT, int DH>
__global__ __launch_bounds__(kNT) void decode_kernel(DecodeArgs a) {
    using Cf = DecRing<MT>;
    constexpr int NST = Cf::NST, L = Cf::L;
    __shared__ __align__(16) uint16_t ring[Cf::NST * Cf::SE];
    __shared__ PhaseSmem<DH> ps;
    __shared__ unsigned s_base;
    __shared__ Tables tb;
    load_tables(a, tb);

    GridBar bar;
    bar.w = a.sync;
    if (threadIdx.x == 0) s_base = ld_sync(a.sync);
    __syncthreads();
    bar.gen = s_base;
    bar.alive = true;
    __syncthreads();

    const int G = gridDim.x;
    const int lm_in = a.lm_in_kernel;
    const int nj = 2 + 4 * a.NL;
    const int nphases = (lm_in ? 4 : 2) + 9 * a.NL;
    if (a.timeline && blockIdx.x == 0 && threadIdx.x == 0)
        a.timeline[(size_t)(nphases - 1) * G + (nphases - 1)] = __builtin_amdgcn_s_memrealtime();
    RingEngine<MT> R;
    R.start(a, ring, &tb);
    int qc = 0;
    const int row = (int)blockIdx.x - a.rows0;   // this workgroup's row in the row phases, if >= 0
    const bool row_wg = row >= 0 && row < a.T;
    AttnArgs at = a.at;
    at.q = a.q;

    // Phases: 0 fc | 1 layer-0 input + plan | per layer l (base 2 + 9l): +0 QKV,
    // +1 RoPE + KV write, +2 attention splits, +3 merge, +4 O, +5 residual +
    // norm, +6 gate/up, +7 down, +8 residual + next norm (or the final norm of
    // the sampled rows) | [LM head | argmax]. A grid barrier after each but the last.
    for (int p = 0; p < nphases; ++p) {
        int kind, l = 0, r = 0;
        if (p == 0) kind = 0;
        else if (p == 1) kind = 1;
        else if (p == 2 + 9 * a.NL) kind = 0;   // LM head
        else if (p == 3 + 9 * a.NL) kind = 9;   // argmax
        else {
            l = (p - 2) / 9;
            r = (p - 2) % 9;
            kind = (r == 0 || r == 4 || r == 6 || r == 7) ? 0 : (r == 1 ? 2 : r == 2 ? 3 : r == 3 ? 4 : r == 5 ? 5 : 6);
        }
        uint16_t* kpl = reinterpret_cast<uint16_t*>(a.kv + (size_t)(2 * l) * a.plane_bytes);
        uint16_t* vpl = reinterpret_cast<uint16_t*>(a.kv + (size_t)(2 * l + 1) * a.plane_bytes);
        int ahead = 0;   // weight stages streamed ahead after this phase's stores
        if (kind == 0) {
            // a projection: job of this phase
            int j;
            if (p == 0) j = 0;
            else if (p == 2 + 9 * a.NL) j = nj - 1;
            else j = 1 + 4 * l + (r == 0 ? 0 : r == 4 ? 1 : r == 6 ? 2 : 3);
            gemm_phase<MT>(a, R, j, qc, ps.xchg);
            // after QKV come RoPE, attention and the merge, which everyone
            // takes part in: nothing is streamed ahead there
            if (!(p >= 2 && p < 2 + 9 * a.NL && r == 0)) ahead = R.prefetch(a, qc);
        } else if (kind == 1) {
            // layer-0 input (one workgroup per row) and the attention split plan
            if (row_wg) layer0_row(a, row, a.sp_fc, ps.red);
            if (blockIdx.x == G - 1) attn_plan_block<true, kPlanMaxC>(a.at);
            ahead = R.prefetch(a, qc);
        } else if (kind == 2) {
            rope_phase(a, uni(tb.jk[l == 0 ? JK_QKV0 : JK_QKV].splits), kpl, vpl);
        } else if (kind == 3) {
            at.kplane = kpl;
            at.vplane = vpl;
            at.out = a.ao + (size_t)l * a.ao_slot;
            const int items = at.sp.max_units * a.Hkv;
            for (int it = blockIdx.x; it < items; it += G) attn_split_item<DH, false, true, kAttnStages>(at, it, ps.at);
        } else if (kind == 4) {
            at.out = a.ao + (size_t)l * a.ao_slot;
            const int waves = a.T * a.Hq;
            for (int w = blockIdx.x * 4 + (threadIdx.x >> 6); w < waves; w += G * 4) attn_merge_wave<DH, 1, true>(at, w);
            ahead = R.prefetch(a, qc);
        } else if (kind == 5) {
            if (row_wg)
                resid_norm_row(a, row, row, a.sp_o, uni_ptr(tb.lp[LP_NORM_POST][l]),
                               a.u + (size_t)(2 * l + 1) * a.u_slot, true, nullptr, nullptr, ps.red);
            ahead = R.prefetch(a, qc);
        } else if (kind == 6) {
            float* snap = a.dbg ? a.dbg + (size_t)(l + 1) * a.T * a.d : nullptr;
            if (l + 1 < a.NL) {
                if (row_wg)
                    resid_norm_row(a, row, row, a.sp_down, uni_ptr(tb.lp[LP_NORM_IN][l + 1]),
                                   a.u + (size_t)(2 * l + 2) * a.u_slot, true, snap, nullptr, ps.red);
            } else {
                // final norm of the K sampled rows of every request, packed for the LM head
                if (row_wg && row < a.R) {
                    int o = a.new_idx[row];
                    if (o < 0 || o >= a.T) {
                        if (threadIdx.x == 0) flag(a.status, PD_STATUS_BAD_ROW);
                        o = 0;
                    }
                    resid_norm_row(a, o, row, a.sp_down, a.norm_final, a.xg, false, nullptr, a.hidden_out, ps.red);
                }
                if (snap && row_wg)
                    resid_norm_row(a, row, row, a.sp_down, a.norm_final, nullptr, false, snap, nullptr, ps.red);
            }
            ahead = R.prefetch(a, qc);
        } else {
            // greedy draft token of every sampled row: argmax over the LM head's partials
            const int ntiles = a.g_lm * 4;
            if (row_wg && row < a.R) {
                const int m = row;
                float bv = -FLT_MAX;
                int bi = INT_MAX;
                for (int t = threadIdx.x; t < ntiles; t += kNT)
                    better_f(bv, bi, ldc<true>(a.amax_v + (size_t)m * ntiles + t),
                             ldc<true>(a.amax_i + (size_t)m * ntiles + t));
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) {
                    const float ov = __shfl_xor(bv, off, kWave);
                    const int oi = __shfl_xor(bi, off, kWave);
                    better_f(bv, bi, ov, oi);
                }
                __syncthreads();
                if ((threadIdx.x & 63) == 0) {
                    ps.red[threadIdx.x >> 6] = bv;
                    reinterpret_cast<int*>(ps.red)[4 + (threadIdx.x >> 6)] = bi;
                }
                __syncthreads();
                if (threadIdx.x == 0) {
                    float v = ps.red[0];
                    int ix = reinterpret_cast<int*>(ps.red)[4];
                    for (int w = 1; w < 4; ++w) better_f(v, ix, ps.red[w], reinterpret_cast<int*>(ps.red)[4 + w]);
                    if (ix == INT_MAX) {
                        flag(a.status, PD_STATUS_BAD_ROW);
                        ix = 0;
                    }
                    a.draft_ids[m] = ix;
                }
            }
        }
        if (p + 1 < nphases) {
            uint64_t* tl = a.timeline ? a.timeline + (size_t)p * G : nullptr;
            // weight stages streamed ahead are the last copies this workgroup
            // issued (after any store of the phase): they may stay in flight
            (void)ahead;
            grid_barrier<L, NST - 1>(bar, a.status, tl, R.npre);
            if (tl && blockIdx.x == G - 1 && threadIdx.x == 0)
                a.timeline[(size_t)(nphases - 1) * G + p] = __builtin_amdgcn_s_memrealtime();
        }
    }
    vm_wait<0>();   // nothing left in flight into LDS when the workgroup ends
}

}  // namespace

}  // namespace pd

namespace pd {

namespace {

// K splits of a 64-column-tile projection: the count (<= 8) that minimises the
// stages of the busiest of G workgroups
int decode_splits(int N, int K, int G) {
    const int ntn = (N + 63) / 64, ksteps = (K + kRS - 1) / kRS;
    long best = -1;
    int sp_best = 1;
    for (int sp = 1; sp <= 8 && sp <= ksteps; ++sp) {
        const int per = (ksteps + sp - 1) / sp;
        if ((sp - 1) * per >= ksteps) continue;   // no empty split
        const long span = (((long)ntn * sp + G - 1) / G) * per;
        if (best < 0 || span < best) { best = span; sp_best = sp; }
    }
    return sp_best;
}

// workgroups taking part: as few as keep every round of items full (a last
// round with few workgroups streams far below the HBM rate)
int decode_grid(long items, int G) {
    if (items <= 0) return 0;
    const long rounds = (items + G - 1) / G;
    return (int)((items + rounds - 1) / rounds);
}

struct DevInfo {
    int cus = 0;
    bool coop = false;
};

DevInfo device_info() {
    static DevInfo cache[64];
    static bool have[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DevInfo{};
    if (!have[dev]) {
        DevInfo d;
        int coop = 0;
        if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) d.cus = 0;
        if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess) coop = 0;
        d.coop = coop != 0;
        cache[dev] = d;
        have[dev] = true;
    }
    return cache[dev];
}

template <int MT, int DH>
int launch_one(const DecodePlan& p, const DecodeArgs& a, hipStream_t s) {
    static int occ = -1;   // resident workgroups per CU (LDS-bound: one)
    if (occ < 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<MT, DH>, kNT, 0) != hipSuccess) n = 0;
        occ = n;
    }
    if (occ < 1) return PD_EINVAL;
    DecodeArgs args = a;
    void* kargs[] = {&args};
    if (hipLaunchCooperativeKernel((const void*)decode_kernel<MT, DH>, dim3(p.grid), dim3(kNT), kargs, 0, s) !=
        hipSuccess)
        return PD_EHIP;
    return hipGetLastError() == hipSuccess ? PD_OK : PD_EHIP;
}

}  // namespace

DecodePlan plan_decode(const pd_model& m, int T, int R, bool fp8) {
    DecodePlan p;
    std::memset(&p, 0, sizeof(p));
    const DevInfo dv = device_info();
    const int G = dv.cus;
    p.ok = !fp8 && dv.coop && G >= 64 && G <= 256 && T >= 1 && T <= 64 && R >= 1 && R <= T &&
           (m.dh == 64 || m.dh == 128) && m.d <= 4096 && m.N <= PD_MAX_LAYERS;
    if (!p.ok) return p;
    p.mt = T <= 16 ? 1 : (T <= 32 ? 2 : 4);
    p.grid = G;
    // one row workgroup per row at the top of the grid; the projections
    // stream on the workgroups below them
    p.rows0 = G - T;
    const int GS = p.rows0;
    // with one activation tile the LM head streams as fast inside the pass;
    // with more, the separate weight-streaming kernel (two column groups per
    // wave, deeper ring) is faster and runs after the pass
    p.lm_in_kernel = p.mt == 1 ? 1 : 0;
    const int qkvw = (m.Hq + 2 * m.Hkv) * m.dh, hd = m.Hq * m.dh;
    p.sp_fc = decode_splits(m.d, m.hidden3, GS);
    p.sp_qkv0 = decode_splits(qkvw, 2 * m.d, GS);
    p.sp_qkv = decode_splits(qkvw, m.d, GS);
    p.sp_o = decode_splits(m.d, hd, GS);
    p.sp_down = decode_splits(m.d, m.F, GS);
    auto grid64 = [&](int N, int sp) { return decode_grid((long)((N + 63) / 64) * sp, GS); };
    p.g_fc = grid64(m.d, p.sp_fc);
    p.g_qkv0 = grid64(qkvw, p.sp_qkv0);
    p.g_qkv = grid64(qkvw, p.sp_qkv);
    p.g_o = grid64(m.d, p.sp_o);
    p.g_gu = decode_grid((m.F + 31) / 32, GS);
    p.g_down = grid64(m.d, p.sp_down);
    p.g_lm = grid64(m.V, 1);
    p.lm_ntiles = p.g_lm * 4;
    size_t ws = 0;
    ws = std::max(ws, (size_t)p.sp_fc * T * m.d);
    ws = std::max(ws, (size_t)std::max(p.sp_qkv0, p.sp_qkv) * T * qkvw);
    ws = std::max(ws, (size_t)std::max(p.sp_o, p.sp_down) * T * m.d);
    p.ws_floats = ws;
    return p;
}

int launch_decode(const DecodePlan& p, const DecodeArgs& a, hipStream_t s) {
    if (!p.ok) return PD_EINVAL;
    if (a.dh == 64) {
        switch (p.mt) {
            case 1: return launch_one<1, 64>(p, a, s);
            case 2: return launch_one<2, 64>(p, a, s);
            case 4: return launch_one<4, 64>(p, a, s);
            default: return PD_EINVAL;
        }
    }
    if (a.dh == 128) {
        switch (p.mt) {
            case 1: return launch_one<1, 128>(p, a, s);
            case 2: return launch_one<2, 128>(p, a, s);
            case 4: return launch_one<4, 128>(p, a, s);
            default: return PD_EINVAL;
        }
    }
    return PD_EINVAL;
}

}  // namespace pd
