// gemm_prefill.hip -- prefill-batch residual-binary GEMM on the fp16 matrix
// cores of gfx950: Y[m][r] = sum_j What[r][j] X[m][j] with
// What[r][j] = sum_k a_k[r][t(j)] (bit ? +1 : -1) ("RaBiT" summary,
// paperlayer.ai, section 4.1: binary cores with per-channel scales;
// "QBB" summary, atlas.scime.ai, "Key results": per-group scales).
//
// With thousands of tokens the layer is a dense contraction: What (the sum
// of the K signed scales, rounded once to fp16) multiplies the fp16
// activations (kept exact) on the fp16 matrix cores, with fp32 accumulation
// and one fp16 rounding of each output.  fp16 rather than bf16: the
// activations stay exact in fp16, and the single rounding of What costs a
// relative error of at most 2^-11 per weight.
//
// Two kernels.  One and two planes (2^K <= 4 values of What per row and
// group) use the second kernel below, which forms What in registers by table
// lookup and stages only activations through LDS.  Three and four planes,
// and shapes whose byte offsets pass 32 bits, use the first, which unpacks
// each weight tile into LDS:
//
// Tiling of the first: a workgroup (8 waves) computes a 256-token x 128-row output tile;
// wave (wm, wn) owns 64 x 64 of it as 4 x 4 MFMA tiles of 16 x 16.  The K
// loop steps 64 columns at a time through double-buffered LDS; the next
// step's activation words and weight bits are requested before the current
// step's MFMAs are issued.  Rows of both LDS tiles are padded to 72 halves
// so that the 16-byte fragment reads of 16 lanes fall in distinct banks.
#include "rbq_device.h"
#include "rbq_kernels.h"

namespace rbq {

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int PF_WAVES = 8;
constexpr int PF_THREADS = PF_WAVES * RBQ_WAVE;
constexpr int BM = 256;            // tokens per tile
constexpr int BN = 128;            // weight rows per tile
constexpr int BK = 64;             // columns per step
constexpr int LDP = BK + 8;        // padded LDS row pitch (halves)

template <int K>
__global__ __launch_bounds__(PF_THREADS, 1) void gemm_prefill_kernel(
    const uint32_t *__restrict__ planes, const uint16_t *__restrict__ scales, int out, int in,
    int group_size, const uint16_t *__restrict__ X, int M, uint16_t *__restrict__ Y) {
    __shared__ __align__(16) _Float16 As[2][BM * LDP];
    __shared__ __align__(16) _Float16 Bs[2][BN * LDP];

    const int tid = threadIdx.x;
    const int lane = tid & (RBQ_WAVE - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / RBQ_WAVE);
    const int wm = wave & 3, wn = wave >> 2;          // 4 x 2 waves
    const int li = lane & 15, lg = lane >> 4;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int words = in >> 5;
    const int G = group_size ? in / group_size : 1;
    const int nsteps = in / BK;

    // ---- global -> register assignments
    // activations: 256 rows x 64 columns = 2048 x 16 bytes; thread: 4 pieces
    // (row = piece / 8, 8 halves at column 8 * (piece % 8))
    int a_row[4], a_col[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int piece = tid + p * PF_THREADS;
        a_row[p] = piece >> 3;
        a_col[p] = (piece & 7) * 8;
    }
    const uint16_t *a_src[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
        a_src[p] = X + (size_t)min(m0 + a_row[p], M - 1) * in + a_col[p];
    // weights: 128 rows x 64 columns; thread: row tid / 4, 16 columns at 16 * (tid % 4)
    const int b_row = tid >> 2, b_q = tid & 3;
    const int b_r = min(n0 + b_row, out - 1);
    const uint32_t *b_src = planes + (size_t)b_r * words + (b_q >> 1);
    const int b_shift = 16 * (b_q & 1);
    const size_t plane_stride = (size_t)out * words;

    uint4 a_reg[4];
    uint32_t b_reg[K];
    uint16_t s_reg[K];
    auto fetch = [&](int step) {
        const int k0 = min(step, nsteps - 1) * BK;
        const int t = group_size ? (k0 + 16 * b_q) / group_size : 0;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            a_reg[p] = *reinterpret_cast<const uint4 *>(a_src[p] + k0);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            b_reg[k] = b_src[k * plane_stride + k0 / 32];
            s_reg[k] = scales[((size_t)k * out + b_r) * G + t];
        }
    };
    // What for 16 columns of one row: sum_k (+-a_k), rounded once to fp16
    auto stash = [&](int step, int buf) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
            *reinterpret_cast<uint4 *>(&As[buf][a_row[p] * LDP + a_col[p]]) = a_reg[p];
        (void)step;
        float sc[K];
#pragma unroll
        for (int k = 0; k < K; ++k)
            sc[k] = h2f(s_reg[k]);
        v8h v0, v1;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float w = 0.0f;
#pragma unroll
            for (int k = 0; k < K; ++k)
                w += ((b_reg[k] >> (b_shift + j)) & 1u) ? sc[k] : -sc[k];
            if (j < 8)
                v0[j] = (_Float16)w;
            else
                v1[j - 8] = (_Float16)w;
        }
        v8h *dst = reinterpret_cast<v8h *>(&Bs[buf][b_row * LDP + 16 * b_q]);
        dst[0] = v0;
        dst[1] = v1;
    };

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

    fetch(0);
    stash(0, 0);
    __syncthreads();
    for (int step = 0; step < nsteps; ++step) {
        const int buf = step & 1;
        fetch(step + 1);           // in flight during the MFMAs (a clamped repeat at the end)
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            v8h af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const v8h *>(
                    &As[buf][(wm * 64 + i * 16 + li) * LDP + ks * 32 + 8 * lg]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *reinterpret_cast<const v8h *>(
                    &Bs[buf][(wn * 64 + j * 16 + li) * LDP + ks * 32 + 8 * lg]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (step + 1 < nsteps)
            stash(step + 1, buf ^ 1);
        __syncthreads();
    }

    // ---- C[i][j] of an MFMA tile sits in lane j + 16*(i/4), register i%4:
    // i = token (A row), j = weight row (B column)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = n0 + wn * 64 + j * 16 + li;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + wm * 64 + i * 16 + 4 * lg + v;
                if (m < M && r < out)
                    Y[(size_t)m * out + r] = f2h(acc[i][j][v]);
            }
        }
}

// ---------------------------------------------------------------------------
// One and two planes: the weights never pass through LDS.
//
// What takes only 2^K values per row (per row and group with group scales):
// with v = b_1 + 2 b_2 the value is sum_k (b_k ? a_k : -a_k), one fp32 sum
// rounded once to fp16, the same value the kernel above writes to LDS.  Each
// lane keeps the four values of its weight row as a byte table (low bytes in
// one register, high bytes in another), and a B fragment of 8 fp16 weights
// comes out of four v_perm_b32 lookups whose selectors are built from the
// sign bits with a few shifts, masks and byte permutes (about 4 VALU
// operations per 2 weights).  Only the activations are staged through LDS,
// which halves the LDS traffic per MFMA compared with unpacking into LDS.
//
// Tiling: a workgroup (4 waves) computes 128 tokens x 256 weight rows; wave w
// owns rows [64 w, 64 w + 64) of it for all 128 tokens, as 4 x 2 tiles of
// v_mfma_f32_32x32x16_f16 (A = activations, B = weights).  The K loop steps
// 64 columns per stage.  Within a stage, lane half h of sub-step ks holds
// columns 32 h + 8 ks + e (e = 0..7) on both operands, so a lane needs byte
// ks of word h of its row's 64-column span -- one 32-bit word per plane and
// stage -- and 16 contiguous bytes of an activation row per sub-step.
// Workgroups are numbered so that each XCD gets a contiguous run of tiles
// (row tiles fastest), so concurrent workgroups on one XCD share activation
// tiles in its L2.
//
// Operands stream into an LDS ring of NB stages by direct global-to-LDS
// loads (global_load_lds_dwordx4 for activations, global_load_lds_dword for
// sign words) issued NB - 1 stages ahead, one load between every few MFMAs
// (issued together at the start of a stage they held the in-order wave back
// from its MFMAs).  One barrier per stage: a wave waits for its own loads of
// the next stage, then the barrier makes every wave's loads visible and frees
// the slot read in the previous stage, which this stage's loads refill.  The
// loads are inline assembly: they have no register results, and the waits
// for them are explicit (the compiler would wait for all of them before
// every LDS read).  The next stage's B fragments are built between this
// stage's MFMAs: the wave issues in order, so VALU work overlaps the matrix
// core only when it sits between the MFMAs.
//
// Activation slot: 128 tokens x 64 columns, 16-byte pieces, token T's piece
// q stored at T * 128 + 16 (q ^ (T & 7) ^ ((T >> 3) & 1)), so that the
// fragment reads of 16 lanes (16 tokens, one piece) hit distinct banks; the
// loads write 1 KB (8 tokens) per wave instruction, lane i the 16 bytes at
// position i.  Sign-word slot: per wave, row block and plane, 64 words, the
// word of lane i at position i.
constexpr int PB_THREADS = 256;
constexpr int PB_BM = 128;             // tokens per tile
constexpr int PB_BN = 256;             // weight rows per tile (64 per wave)
constexpr int PB_BK = 64;              // columns per stage

typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int PR_SLOT_A = PB_BM * PB_BK * 2;   // 16 KB

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// The two loads below set M0 themselves; nothing else in the kernels that
// use them reads M0 (no LDS-DMA builtins, message or relative-move
// instructions), so the compiler keeps no value there.
// 16 bytes from base + voff to LDS [m0 + 16 lane]
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(m0)
                 : "memory");
}
// 4 bytes from base + voff to LDS [m0 + 4 lane]
__device__ __forceinline__ void dma4(const void *base, uint32_t voff, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(m0)
                 : "memory");
}

template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int K, bool GROUPED, int NB>
__global__ __launch_bounds__(PB_THREADS, 2) void gemm_prefill_ring_kernel(
    const uint32_t *__restrict__ planes, const uint16_t *__restrict__ scales, int out, int in,
    int group_size, const uint16_t *__restrict__ X, int M, uint16_t *__restrict__ Y, int tiles_n,
    int total) {
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr int SLOT_B = 4 * 2 * K * 256;          // sign words of the 4 waves
    constexpr int SLOT = PR_SLOT_A + SLOT_B;
    constexpr int PD = NB - 1;                       // stages in flight
    static_assert(NB >= 3 && (NB - 1) * (4 + 2 * K) < 64, "ring depth");
    constexpr int PER_STAGE = 4 + 2 * K;             // loads per thread and stage

    const int tid = threadIdx.x;
    const int lane = tid & (RBQ_WAVE - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / RBQ_WAVE);
    const int l32 = lane & 31, h = lane >> 5;

    int id = blockIdx.x;
    const int per = total >> 3;
    if (id < per * 8)
        id = (id & 7) * per + (id >> 3);
    const int tm = id / tiles_n, tn = id - tm * tiles_n;
    const int m0 = tm * PB_BM, n0 = tn * PB_BN;
    const int words = in >> 5;
    const int nst = in / PB_BK;
    const int G = GROUPED ? in / group_size : 1;
    const int spg = GROUPED ? group_size / PB_BK : 1;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));

    // activation loads: wave block 4 wave + j holds tokens 8 (4 wave + j) + lane / 8
    uint32_t a_voff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = 8 * (4 * wave + j) + (lane >> 3);
        const int q = (lane & 7) ^ (t & 7) ^ ((t >> 3) & 1);
        a_voff[j] = (uint32_t)(min(m0 + t, M - 1) * in + 8 * q) * 2u;
    }
    int rowc[2];
    uint32_t b_voff[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        rowc[b] = min(n0 + 64 * wave + 32 * b + l32, out - 1);
        b_voff[b] = (uint32_t)(rowc[b] * words + h) * 4u;
    }
    const uint32_t pstride_b = (uint32_t)out * (uint32_t)words * 4u;

    // load q of a stage into ring slot `at`: q < 4 activations (block
    // 4 wave + q), then the sign words (row block, plane)
    auto issue_piece = [&](int st, int at, int q) {
        const uint32_t slot = lds0 + (uint32_t)(at % NB) * SLOT;
        if (q < 4) {
            dma16(X, a_voff[q] + (uint32_t)st * (PB_BK * 2), slot + (uint32_t)(4 * wave + q) * 1024u);
        } else {
            const int b = (q - 4) / K, k = (q - 4) % K;
            dma4(planes, b_voff[b] + k * pstride_b + (uint32_t)st * 8u,
                 slot + PR_SLOT_A + (uint32_t)((wave * 2 + b) * K + k) * 256u);
        }
    };
    auto issue = [&](int st) {
#pragma unroll
        for (int q = 0; q < PER_STAGE; ++q)
            issue_piece(min(st, nst - 1), st, q);
    };

    uint32_t plo[2], phi[2];
    auto make_tables = [&](int t) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            float a[K];
#pragma unroll
            for (int k = 0; k < K; ++k)
                a[k] = h2f(scales[((size_t)k * out + rowc[b]) * G + t]);
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float w = 0.0f;
#pragma unroll
                for (int k = 0; k < K; ++k)
                    w += ((v >> k) & 1) ? a[k] : -a[k];
                const uint32_t hv = f2h(w);
                lo |= (hv & 0xFFu) << (8 * v);
                hi |= (hv >> 8) << (8 * v);
            }
            plo[b] = lo;
            phi[b] = hi;
        }
    };

    // fragment read offsets: token i * 32 + l32, piece 4 h + ks (swizzled)
    const int swz = (l32 & 7) ^ ((l32 >> 3) & 1);
    uint32_t a_rd[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        a_rd[ks] = (uint32_t)(l32 * 128 + 16 * ((4 * h + ks) ^ swz));

    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][b][r] = 0.0f;

    // B fragments of a stage from its sign words: dword p of sub-step ks
    // holds the weights of columns 32 h + 8 ks + 2p and + 2p + 1.
    auto build = [&](int st, v4u (&bf)[2][4]) {
        const unsigned char *slot = lds + (st % NB) * SLOT;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint32_t *sw = reinterpret_cast<const uint32_t *>(slot + PR_SLOT_A) + (wave * 2 + b) * K * 64;
            const uint32_t w1 = sw[lane], w2 = K > 1 ? sw[64 + lane] : 0u;
            // 2-bit table index v of every even column (z) and odd column (zo)
            const uint32_t z = (w1 & 0x55555555u) | ((w2 & 0x55555555u) << 1);
            const uint32_t zo = ((w1 >> 1) & 0x55555555u) | (w2 & 0xAAAAAAAAu);
            const uint32_t y01 = __builtin_amdgcn_perm(zo, z, 0x05040100u);   // [z.b0 z.b1 zo.b0 zo.b1]
            const uint32_t y23 = __builtin_amdgcn_perm(zo, z, 0x07060302u);   // [z.b2 z.b3 zo.b2 zo.b3]
#pragma unroll
            for (int p = 0; p < 4; ++p) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const uint32_t ym = ((half ? y23 : y01) >> (2 * p)) & 0x03030303u;
                    const uint32_t ym4 = ym | 0x04040404u;
                    // selectors [v, v + 4, v', v' + 4] of the two sub-steps
                    const uint32_t s0 = __builtin_amdgcn_perm(ym4, ym, 0x06020400u);
                    const uint32_t s1 = __builtin_amdgcn_perm(ym4, ym, 0x07030501u);
                    bf[b][2 * half][p] = __builtin_amdgcn_perm(phi[b], plo[b], s0);
                    bf[b][2 * half + 1][p] = __builtin_amdgcn_perm(phi[b], plo[b], s1);
                }
            }
        }
    };

#pragma unroll
    for (int st = 0; st < PD; ++st)
        issue(st);   // (past the last stage: the last stage again, into an unused slot)
    make_tables(0);
    // stage 0 landed (PD - 1 younger stages may be in flight)
    vm_wait_barrier<(PD - 1) * PER_STAGE>();
    // One stage: MFMAs on the fragments built in the previous stage, and
    // between them, one piece at a time, the next stage's fragments (the
    // wave issues in order, so the build overlaps the matrix core only when
    // its instructions sit between the MFMAs; sched_barrier keeps them there).
    auto stage = [&](int st, const v4u (&cur)[2][4], v4u (&nxt)[2][4]) {
        // stage st + 1 landed; every wave is done with stage st - 1, whose
        // slot the loads of stage st + PD refill
        // (every stage issues PER_STAGE loads, so PD - 2 younger stages)
        vm_wait_barrier<(PD - 2) * PER_STAGE>();
        // New group tables before the next loads are issued: the compiler
        // waits for its scale loads with vmcnt(0), which then drains only the
        // one stage still in flight.
        if (GROUPED && st + 1 < nst && (st + 1) % spg == 0)
            make_tables((st + 1) / spg);
        // the loads of stage st + PD go out one at a time between the MFMAs
        // below; past the last stage they repeat it into a free slot
        const int ld_st = min(st + PD, nst - 1), ld_at = st + PD;
        const unsigned char *slot = lds + (st % NB) * SLOT;
        const unsigned char *nslot = lds + (min(st + 1, nst - 1) % NB) * SLOT;
        // sign words of the next stage (the last stage rereads its own, unused)
        uint32_t w1[2], w2[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint32_t *sw = reinterpret_cast<const uint32_t *>(nslot + PR_SLOT_A) + (wave * 2 + b) * K * 64;
            w1[b] = sw[lane];
            w2[b] = K > 1 ? sw[64 + lane] : 0u;
        }
        v8h af[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[0][i] = *reinterpret_cast<const v8h *>(slot + a_rd[0] + i * 4096);
        uint32_t y01[2], y23[2];
        // unit u of the build: u = 0, 1 index words of row block u; u >= 2:
        // table lookups (row block, p, half) for two sub-steps
        auto unit = [&](int u) {
            if (u < 2) {
                const int b = u;
                const uint32_t z = (w1[b] & 0x55555555u) | ((w2[b] & 0x55555555u) << 1);
                const uint32_t zo = ((w1[b] >> 1) & 0x55555555u) | (w2[b] & 0xAAAAAAAAu);
                y01[b] = __builtin_amdgcn_perm(zo, z, 0x05040100u);   // [z.b0 z.b1 zo.b0 zo.b1]
                y23[b] = __builtin_amdgcn_perm(zo, z, 0x07060302u);   // [z.b2 z.b3 zo.b2 zo.b3]
            } else if (u < 18) {
                const int b = (u - 2) & 1, p = ((u - 2) >> 1) & 3, half = (u - 2) >> 3;
                const uint32_t ym = ((half ? y23[b] : y01[b]) >> (2 * p)) & 0x03030303u;
                const uint32_t ym4 = ym | 0x04040404u;
                // selectors [v, v + 4, v', v' + 4] of the two sub-steps
                const uint32_t s0 = __builtin_amdgcn_perm(ym4, ym, 0x06020400u);
                const uint32_t s1 = __builtin_amdgcn_perm(ym4, ym, 0x07030501u);
                nxt[b][2 * half][p] = __builtin_amdgcn_perm(phi[b], plo[b], s0);
                nxt[b][2 * half + 1][p] = __builtin_amdgcn_perm(phi[b], plo[b], s1);
            }
        };
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    af[(ks + 1) & 1][i] = *reinterpret_cast<const v8h *>(slot + a_rd[ks + 1] + i * 4096);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = j >> 1, b = j & 1;
                acc[i][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    af[ks & 1][i], __builtin_bit_cast(v8h, cur[b][ks]), acc[i][b], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                const int u = ks * 8 + j;
                if (u >= 4 && u < 22)
                    unit(u - 4);   // the first MFMAs cover the LDS latency of the words
                if (u % 4 == 1 && u / 4 < PER_STAGE)
                    issue_piece(ld_st, ld_at, u / 4);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the fragments count as used here, so the build is not sunk into
        // the next stage (next to its use, after this stage's MFMAs)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                asm volatile("" : "+v"(nxt[b][ks]));
    };

    v4u bfa[2][4], bfb[2][4];
    build(0, bfa);
    int st = 0;
    for (; st + 1 < nst; st += 2) {
        stage(st, bfa, bfb);
        stage(st + 1, bfb, bfa);
    }
    if (st < nst)
        stage(st, bfa, bfb);
    // no LDS loads outstanding when the waves end
    vm_wait_barrier<0>();

#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int row = n0 + 64 * wave + 32 * b + l32;
        if (row < out) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                    if (m < M)
                        Y[(size_t)m * out + row] = f2h(acc[i][b][r]);
                }
        }
    }
}

int prefill_num_cus() {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
    }
    return cus;
}

// Ring depth: 4 stages (80 KB of LDS) when every workgroup has a compute unit
// to itself, 3 (60 KB) when two share one, which measured faster there.
template <int K, bool GROUPED>
hipError_t launch_ring(const uint32_t *planes, const uint16_t *scales, int out, int in,
                       int group_size, const uint16_t *X, int M, uint16_t *Y, hipStream_t st) {
    const int tiles_n = (out + PB_BN - 1) / PB_BN;
    const int tiles_m = (M + PB_BM - 1) / PB_BM;
    const long long total = (long long)tiles_n * tiles_m;
    if (total > 0x7FFFFFFFLL)
        return hipErrorInvalidValue;
    const int nb = total > prefill_num_cus() ? 3 : 4;
    const size_t lds = (size_t)nb * (PR_SLOT_A + 4 * 2 * K * 256);
    if (nb == 3)
        hipLaunchKernelGGL((gemm_prefill_ring_kernel<K, GROUPED, 3>), dim3((unsigned)total), dim3(PB_THREADS),
                           lds, st, planes, scales, out, in, group_size, X, M, Y, tiles_n, (int)total);
    else
        hipLaunchKernelGGL((gemm_prefill_ring_kernel<K, GROUPED, 4>), dim3((unsigned)total), dim3(PB_THREADS),
                           lds, st, planes, scales, out, in, group_size, X, M, Y, tiles_n, (int)total);
    return hipGetLastError();
}

template <int K>
hipError_t launch_k(const uint32_t *planes, const uint16_t *scales, int out, int in,
                    int group_size, const uint16_t *X, int M, uint16_t *Y, hipStream_t st) {
    dim3 grid((out + BN - 1) / BN, (M + BM - 1) / BM);
    hipLaunchKernelGGL(gemm_prefill_kernel<K>, grid, dim3(PF_THREADS), 0, st, planes, scales,
                       out, in, group_size, X, M, Y);
    return hipGetLastError();
}

}  // namespace

bool prefill_supports(int in, int K, int group_size, int M) {
    return K >= 1 && K <= 4 && in % BK == 0 && in > 0 && M >= 1 && (M + BM - 1) / BM <= 65535 &&
           (group_size == 0 || group_size % BK == 0);
}

hipError_t launch_gemm_prefill(const uint32_t *planes, const uint16_t *scales, int out, int in,
                               int K, int group_size, const uint16_t *X, int M, uint16_t *Y,
                               hipStream_t st) {
    if (!prefill_supports(in, K, group_size, M))
        return hipErrorInvalidValue;
    // 32-bit byte offsets in the bit-unpacking kernels
    const bool small = (size_t)M * in < (1ull << 31) && (size_t)out * (in / 32) * K < (1ull << 30);
    if (K <= 2 && small) {
        if (group_size == 0)
            return K == 1 ? launch_ring<1, false>(planes, scales, out, in, 0, X, M, Y, st)
                          : launch_ring<2, false>(planes, scales, out, in, 0, X, M, Y, st);
        return K == 1 ? launch_ring<1, true>(planes, scales, out, in, group_size, X, M, Y, st)
                      : launch_ring<2, true>(planes, scales, out, in, group_size, X, M, Y, st);
    }
    switch (K) {
    case 1: return launch_k<1>(planes, scales, out, in, group_size, X, M, Y, st);
    case 2: return launch_k<2>(planes, scales, out, in, group_size, X, M, Y, st);
    case 3: return launch_k<3>(planes, scales, out, in, group_size, X, M, Y, st);
    case 4: return launch_k<4>(planes, scales, out, in, group_size, X, M, Y, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace rbq
