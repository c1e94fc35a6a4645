// gemv_program.hip -- a list of residual-binary GEMVs (one token) run by one
// persistent launch.
//
// Each op is y = sum_k a_k (.) (B_k x) with per-row scales ("RaBiT" summary,
// paperlayer.ai, sections 4.1 and 4.2; D "GPU implementation": 32 columns per
// word), computed as in the flat kernel: x quantised once per op to
// q = round(x 2^sh) split into three signed bytes, the masked weight words
// w & (0x01010101 << s) as the A operand of v_mfma_i32_16x16x64_i8, and
// y = sum_k a_k (2 S_k - sum q) 2^-sh.
//
// Why one launch.  A decode step is a chain of GEMVs over weights that do
// not depend on the activations.  Launched one by one, every GEMV pays the
// launch latency and the ramp of its first HBM requests (about 2 us), which
// at Llama-2-7B sizes (4-23 MB per GEMV) is a third of its time.  Here one
// 16-wave workgroup per compute unit walks the whole list:
//   * 12 stream waves keep a ring of 16-byte weight loads in flight that
//     runs on from one op into the next, so HBM stays busy across op
//     boundaries.  In the row layout a load covers 64 bytes of 16 rows, half
//     a 128-byte line of each; the wave's next unit reads the other halves,
//     so the loads are ordinary cached ones (with the non-temporal hint the
//     FETCH_SIZE counter showed 1.8 times the plane bytes read from HBM,
//     without it 1.07 times).  In the tile layout (RBQ_LAYOUT_TILES) a load
//     is one contiguous 1 KB block, 8 whole lines, which HBM serves faster;
//   * 4 image waves build each op's activation image (x quantised into LDS,
//     laid out as the MFMA B operand; two buffers, so op i+1's image is
//     built while op i streams), and finish each op: the int32 partial sums
//     of a 16-row tile meet in LDS, one image thread per row applies the
//     scales and writes y;
//   * an op may wait for an earlier op (its x is that op's y, as in a
//     decoder layer): the image waves of every workgroup, after writing their
//     rows of the earlier op's y with device-coherent stores, add 1 to that
//     op's counter in global memory; the waiting op's image is built once
//     the counter reaches the number of workgroups, from device-coherent
//     loads of x.  Weight loads never wait, so the ring keeps streaming the
//     next op's weights meanwhile.
// A program without waits runs a kernel built without the waiting code, and
// a program whose ops all read the tile layout one without the row layout's
// addressing (the per-load choice between the two layouts cost that layout
// its gain: 420 us per step against 408 us for the decode step).
// Every wait is bounded (0.2 s of the real-time clock); a wait that runs out sets
// RBQ_STATUS_PROGRAM_TIMEOUT in the status word and the kernel still runs to
// its end.  The waits across workgroups need all workgroups resident: one
// per compute unit, as launched (the LDS each takes leaves room for one).
#include <stddef.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "rbq.h"
#include "rbq_device.h"
#include "rbq_kernels.h"

namespace rbq {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

constexpr int PG_WAVES = 16;
constexpr int PG_THREADS = PG_WAVES * RBQ_WAVE;
constexpr int PG_PREP = 4;                                 // image waves
constexpr int PG_PREP_THREADS = PG_PREP * RBQ_WAVE;
constexpr int PG_STREAM = PG_WAVES - PG_PREP;              // stream waves
constexpr int TILE_ROWS = 16;
constexpr int CHUNK_WORDS = 16;                            // 512 columns
constexpr int NLIMB = 3;                                   // MFMA columns per token: its 3 limbs
// image bytes per chunk for ops of mt tokens (3 mt MFMA columns; +64: other banks)
__host__ __device__ constexpr int img_chunk_bytes(int mt) { return 8 * 4 * 16 * NLIMB * mt + 64; }
constexpr int PG_ROWS_PER_THREAD = 3;                      // rows of one op that an image thread finishes, at most
constexpr int PG_MAX_TILES = PG_ROWS_PER_THREAD * PG_PREP_THREADS / TILE_ROWS;   // 48 tiles of one op per workgroup
constexpr int PG_MAX_XU = 4;                               // half-words (16 columns) per image thread
// half-words (16 columns) per image thread and token for ops of mt tokens;
// the widest input of such ops is that times 256 threads times 16 columns:
// 16384 (one token), 12288 (two), 4096 (four)
__host__ __device__ constexpr int max_xu(int mt) { return mt == 1 ? PG_MAX_XU : mt == 2 ? 3 : 1; }
__host__ __device__ constexpr int max_in_of(int mt) { return max_xu(mt) * PG_PREP_THREADS * 16; }
constexpr int PG_MAX_CHUNKS = PG_MAX_XU * PG_PREP_THREADS / (2 * CHUNK_WORDS);   // 32: in <= 16384
constexpr uint64_t PG_WAIT_TICKS = 20000000;               // bound of every wait: 0.2 s of the
                                                           // 100 MHz real-time clock (never reached)
constexpr size_t PG_MIN_LDS = 96 * 1024;                   // one workgroup per compute unit
constexpr int PG_SLOTS = 4;                                // ops in flight: partial sums, scales, sums
constexpr uint32_t PG_NO_NEXT = 0xFFFu;                    // an op's group has no later op (> RBQ_PROGRAM_MAX_OPS)
static_assert(RBQ_PROGRAM_MAX_OPS < (int)PG_NO_NEXT, "op links take 12 bits");
#ifndef RBQ_PROGRAM_GROUPS
#define RBQ_PROGRAM_GROUPS 8                               // op groups of programs without waits, at most (1, 2, 4 or 8)
#endif
constexpr uint32_t PG_MAGIC = 0x52425150u;                 // "RBQP"
constexpr int PG_MAX_G = PG_MAX_CHUNKS * 4;                // 128-column groups of the widest input

// flags of an op
constexpr uint32_t PF_SILU = 1u;       // (gate, up) row pairs -> silu(gate) * up
constexpr uint32_t PF_X_SHARED = 2u;   // x is written by an earlier op of the program
constexpr uint32_t PF_SIGNAL = 4u;     // a later op waits for this one
constexpr uint32_t PF_Y_SHARED = 8u;   // y is read (or written again) by a later op
constexpr uint32_t PF_REUSE = 32u;     // same x as the op before: its image is used again
constexpr uint32_t PF_TILES = 64u;     // planes in the tile layout (1 KB per 16-row, 512-column unit)
constexpr int PF_WROT_SHIFT = 8;       // bits 8..11: rotation of the stream waves over the units
constexpr int PF_GRP_SHIFT = 12;       // bits 12..14: the op group (of the workgroups) that runs the op

// One op in device memory (64 bytes).
struct ProgOp {
    const uint32_t *planes;
    const uint16_t *scales;
    const uint16_t *x;
    uint16_t *y;
    int32_t out, in;
    int16_t wait_for;     // earlier op this one waits for (-1: none)
    int16_t free_after;   // the last earlier op of the group to finish before this op is built: the
                          // one whose image shares LDS bytes with its own, or PG_SLOTS places back
                          // (whose slot it takes) (-1: none)
    uint32_t flags;
    int32_t trot;         // rotation of the group's workgroups that take one more tile (bits 0..15) |
                          // the op's place in its group's sequence (bits 16..)
    uint32_t split;       // tiles / G (bits 0..7) | tiles % G (bits 8..19): the tile split, precomputed |
                          // the next op of the same group (bits 20..31; PG_NO_NEXT after its last)
    uint32_t nch_img;     // 512-column chunks (bits 0..7) | image offset in the arena / 16 (bits 8..)
    uint32_t magic;       // ceil(2^21 / chunks): unit -> (tile, chunk) by a multiply and a shift
};
static_assert(sizeof(ProgOp) == 64, "op layout");

// Program image: header, ops, then the unit count of every (workgroup,
// stream wave) over the whole program.
struct ProgHeader {
    uint32_t magic;
    int32_t n_ops;
    int32_t K;
    int32_t grid;
    uint32_t lds_bytes;
    uint32_t checksum;
    int32_t arena_bytes;   // LDS bytes of the image arena
    int32_t kind;          // PK_* bits: which kernel runs the program
};
static_assert(sizeof(ProgHeader) == 32, "header layout");

constexpr int32_t PK_WAITS = 1;        // some op waits for another: the kernel with the waits
constexpr int32_t PK_TILES = 2;        // every op reads the tile layout
constexpr int32_t PK_GROUP = 4;        // g128 ops (scales per 128-column group, in the scale tile layout)
constexpr int PK_P_SHIFT = 4;          // bits 4..7: P, the number of op groups (1, 2, 4 or 8)
constexpr int32_t PK_P_MASK = 15 << PK_P_SHIFT;
constexpr int PK_T_SHIFT = 8;          // bits 8..15: tiles of an op per workgroup at most (the LDS slots' size)
constexpr int32_t PK_T_MASK = 255 << PK_T_SHIFT;
constexpr int PK_MT_SHIFT = 16;        // bits 16..17: log2 of the tokens every op carries (1, 2 or 4)
constexpr int32_t PK_MT_MASK = 3 << PK_MT_SHIFT;

// The kernel's fixed LDS (its size is known to the host, which gives the
// image arena what remains of the compute unit's LDS).  Programs of g128 ops
// (GROUP) also keep the sum of q over every 128-column group of each x.
template <int K, bool GROUP, int MT = 1>
struct PgShared {
    int img_cnt;                              // image waves' publications: 4 per op
    int sdone[PG_SLOTS];                      // stream waves done with an op, by op slot (i % PG_SLOTS)
    int isync;                                // phases of the image waves' barrier
    int abort_flag;                           // a wait ran out: the rest runs without waiting
    int last_wg;                              // this workgroup is the last to finish the run
    uint32_t wmax[PG_SLOTS][MT][PG_PREP];
    double wsum[PG_SLOTS][MT][PG_PREP];             // sums of q per token (exact: integers below 2^53)
    int shs[PG_SLOTS][MT];
    uint16_t sc_lds[PG_SLOTS][GROUP ? 1 : K][PG_ROWS_PER_THREAD * PG_PREP_THREADS];   // scales of the rows finished
    int gsum[PG_SLOTS][GROUP ? PG_MAX_G : 1];         // g128: sum of q over each group (|sum| < 2^30)
};

// LDS ints per tile of an op slot of partial sums: per-row ops add int32
// tile sums [tile][plane][limb][row]; g128 ops store fp32 [tile][stream
// wave][row].  A program's slots hold its largest op's tiles per workgroup.
__host__ __device__ constexpr int red_tile_ints(int K, bool group, int mt = 1) {
    return (group ? PG_STREAM : K * NLIMB * mt) * TILE_ROWS;
}

// Op counters: each op's count of finished workgroups is split over
// PG_CSPLIT words (workgroup b adds to word b % PG_CSPLIT), each on its own
// 128-byte line, so that 256 workgroups do not all contend for one address;
// a waiter adds the words up.  The run's own count of finished workgroups
// follows the ops' counters.
constexpr int PG_CSPLIT = 8;
constexpr int PG_CPAD = 32;                                // ints per 128-byte line
__host__ __device__ inline size_t counter_index(int j, int c) { return ((size_t)j * PG_CSPLIT + c) * PG_CPAD; }
__device__ inline int *op_counter(int *counters, int j, int c) { return counters + counter_index(j, c); }

// LDS of one compute unit available to a workgroup (160 KB on gfx950; the
// same when no device is visible, for host-only checks).
size_t program_lds_limit() {
    static size_t lim = 0;
    if (lim == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0)
            v = 160 * 1024;
        lim = (size_t)v;
    }
    return lim;
}

// Dynamic LDS a program may take: the limit less the kernel's fixed LDS
// (and 256 bytes for its alignment).
size_t program_dynamic_lds(int K, bool group, int mt = 1) {
    const size_t fixed = group ? (K == 2 ? sizeof(PgShared<2, true>) : sizeof(PgShared<4, true>))
                               : mt == 4 ? sizeof(PgShared<2, false, 4>)
                               : mt == 2 ? sizeof(PgShared<2, false, 2>)
                                         : (K == 1 ? sizeof(PgShared<1, false>) : sizeof(PgShared<2, false>));
    return program_lds_limit() - fixed - 256;
}

size_t program_counter_ints(int n_ops) { return counter_index(n_ops, 0) + 1; }

size_t image_bytes(int n_ops, int grid) {
    return sizeof(ProgHeader) + (size_t)n_ops * sizeof(ProgOp) + (size_t)grid * PG_STREAM * sizeof(int32_t);
}

int program_num_cus() {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
    }
    return cus;
}

// tiles [t0, t0 + ntl) of an op taken by workgroup b of G: base = T / G
// each, and one more for the extra = T % G workgroups starting at the op's
// rotation (the divisions are done on the host: without an integer divider
// each costs dozens of scalar instructions, per op and wave)
__host__ __device__ inline void op_tiles(int base, int extra, int trot, int b, int G, int &t0, int &ntl) {
    int bb = b - trot;
    bb += bb < 0 ? G : 0;
    ntl = base + (bb < extra ? 1 : 0);
    t0 = bb * base + (bb < extra ? bb : extra);
}

// units [u0, u1) of stream wave sw among the U (tile, chunk) units of a workgroup
__host__ __device__ inline void op_units(int U, int wrot, int sw, int &u0, int &u1) {
    int s = sw + wrot;
    s -= s >= PG_STREAM ? PG_STREAM : 0;
    u0 = (s * U) / PG_STREAM;
    u1 = ((s + 1) * U) / PG_STREAM;
}

// LDS waits (relaxed reads: writers release their LDS stores before they
// count, LDS is coherent within the compute unit).  False when the wait ran
// out or an earlier one did (abort_flag).
// A waiting wave sleeps between polls (s_sleep 4: 256 clocks); every
// producer ends with s_wakeup, which wakes the sleeping waves of its
// workgroup at once.  Polling without sleeping took issue slots and LDS
// bandwidth from the waves doing the work.
__device__ __forceinline__ void wake_workgroup() { asm volatile("s_wakeup" ::: "memory"); }

__device__ __forceinline__ bool lds_wait_ge(int *counter, int target, int *abort_flag) {
    if (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target)
        return true;
    const uint64_t deadline = __builtin_amdgcn_s_memrealtime() + PG_WAIT_TICKS;
    for (int it = 1;; ++it) {
        __builtin_amdgcn_s_sleep(4);
        if (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target)
            return true;
        if ((it & 15) == 0 && (__hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) ||
                               __builtin_amdgcn_s_memrealtime() > deadline))
            return false;
    }
}

__device__ __forceinline__ int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }

// x plus x of the lane CTRL names within the row of 16 lanes (0 past the row's edge)
template <int CTRL>
__device__ __forceinline__ int dpp_row_add_i32(int x) {
    return x + __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_row_add_f32(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF,
                                                                      0xF, false));
}

template <class T>
__device__ __forceinline__ T *rflp(T *p) {
    const uint64_t u = (uint64_t)(uintptr_t)p;
    const uint32_t lo = (uint32_t)rfl((int)(uint32_t)u), hi = (uint32_t)rfl((int)(uint32_t)(u >> 32));
    return reinterpret_cast<T *>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

// Pointers into global memory.  Read back from LDS a pointer is generic,
// and generic (flat) loads count against the LDS wait counter as well: every
// wait for an LDS read would then also wait for the weight loads in flight.
#define GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ GLOBAL T *gptr(T *p) {
    return (GLOBAL T *)p;
}

// The fields of op i (uniform across the wave: scalar registers).
struct OpView {
    GLOBAL const uint32_t *planes;
    GLOBAL const uint16_t *scales;
    GLOBAL const uint16_t *x;
    GLOBAL uint16_t *y;
    int out, in, wait_for, base, extra, nchunks, trot, wrot, free_after, img_off;
    int grp, lpos;        // the op's group, and its place in the group's sequence (its slot: lpos % PG_SLOTS)
    int next;             // the group's next op (>= n_ops after its last)
    uint32_t flags, magic;
};

// The device copy of the program image is only read during a run, so the op
// descriptors come in by scalar loads through the scalar cache, off the
// vector memory and LDS queues.  (Read field by field from an LDS copy of
// the table, one descriptor took 400 ns while the stream waves kept LDS
// busy, on the critical path of every op: the step ran 2-3 % slower.)
__device__ __forceinline__ OpView op_view(const ProgOp *table, int i) {
    typedef const __attribute__((address_space(4))) uint32_t CU32;
    CU32 *w = (CU32 *)(table + rfl(i));
    uint32_t q[16];
#pragma unroll
    for (int e = 0; e < 16; ++e)
        q[e] = w[e];
    auto p64 = [&](int e) { return (uintptr_t)(((uint64_t)q[e + 1] << 32) | q[e]); };
    static_assert(offsetof(ProgOp, out) == 32 && offsetof(ProgOp, wait_for) == 40 && offsetof(ProgOp, flags) == 44 &&
                      offsetof(ProgOp, trot) == 48 && offsetof(ProgOp, split) == 52 &&
                      offsetof(ProgOp, nch_img) == 56 && offsetof(ProgOp, magic) == 60,
                  "op fields read by word");
    OpView v;
    v.planes = gptr(reinterpret_cast<const uint32_t *>(p64(0)));
    v.scales = gptr(reinterpret_cast<const uint16_t *>(p64(2)));
    v.x = gptr(reinterpret_cast<const uint16_t *>(p64(4)));
    v.y = gptr(reinterpret_cast<uint16_t *>(p64(6)));
    v.out = (int)q[8];
    v.in = (int)q[9];
    v.wait_for = (int)(int16_t)(q[10] & 0xFFFFu);
    v.free_after = (int)(int16_t)(q[10] >> 16);
    v.flags = q[11];
    v.trot = (int)(q[12] & 0xFFFFu);
    v.lpos = (int)(q[12] >> 16);
    v.base = (int)(q[13] & 255u);
    v.extra = (int)((q[13] >> 8) & 0xFFFu);
    v.next = (int)(q[13] >> 20);
    v.nchunks = (int)(q[14] & 255u);
    v.img_off = (int)(q[14] >> 8) * 16;
    v.magic = q[15];
    v.wrot = (int)((v.flags >> PF_WROT_SHIFT) & 15u);
    v.grp = (int)((v.flags >> PF_GRP_SHIFT) & 7u);
    return v;
}

// MT: tokens per op (1, or 2 or 4 for programs of several-token per-row ops
// on the tile layout without waits); the MFMA columns 3m .. 3m + 2 hold
// token m's limbs (12 of the 16 columns with four tokens).
template <int K, int RING, bool WAITS, bool TILES, bool GROUP, int MT = 1>
__global__ __launch_bounds__(PG_THREADS, 1) void gemv_program_kernel(
    const ProgHeader *__restrict__ hdr, int n_ops, uint32_t checksum, int *__restrict__ counters,
    int32_t *__restrict__ status) {
    static_assert(MT == 1 || ((MT == 2 || MT == 4) && !GROUP && !WAITS && TILES),
                  "several-token ops: per-row, tiled, no waits");
    constexpr int NC = NLIMB * MT;                  // MFMA columns in use
    constexpr int IMG_CHUNK = img_chunk_bytes(MT);
    constexpr int XU = max_xu(MT);
    extern __shared__ __align__(16) unsigned char lds[];
    __shared__ PgShared<K, GROUP, MT> sh;
    int &img_cnt = sh.img_cnt;
    int *sdone = sh.sdone;
    int &isync = sh.isync;
    int &abort_flag = sh.abort_flag;
    auto &wmax = sh.wmax;
    auto &wsum = sh.wsum;
    auto &shs = sh.shs;
    auto &sc_lds = sh.sc_lds;
    auto &gsum = sh.gsum;

    if (hdr->magic != PG_MAGIC || hdr->n_ops != n_ops || hdr->checksum != checksum || hdr->K != K ||
        hdr->grid != (int)gridDim.x) {
        if (threadIdx.x == 0 && status != nullptr)
            __hip_atomic_fetch_or(status, (int)RBQ_STATUS_PROGRAM_MISMATCH, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const ProgOp *__restrict__ ops_g = reinterpret_cast<const ProgOp *>(hdr + 1);
    const int32_t *__restrict__ wave_units = reinterpret_cast<const int32_t *>(ops_g + n_ops);

    const int tid = threadIdx.x;
    const int lane = tid & (RBQ_WAVE - 1);
    const int wave = rfl(tid / RBQ_WAVE);
    const int li = lane & 15, lg = lane >> 4;
    const int G = gridDim.x;
    const int b = blockIdx.x;
    // op groups: this workgroup is number bl of the Gl workgroups of group mygrp
    const int P = (hdr->kind & PK_P_MASK) >> PK_P_SHIFT;
    const int Gl = G / P;
    const int mygrp = b / Gl, bl = b - mygrp * Gl;
    // tiles [t0, t0 + ntl) of an op taken by this workgroup (none for another group's op)
    auto my_tiles = [&](const OpView &op, int &t0, int &ntl) {
        if (op.grp != mygrp) {
            t0 = 0;
            ntl = 0;
        } else {
            op_tiles(op.base, op.extra, op.trot, bl, Gl, t0, ntl);
        }
    };
    // LDS: image arena, 16 zero bytes, partial sums [PG_SLOTS][max_tiles][K][NC][16]
    const int pad = hdr->arena_bytes;
    int *red0 = reinterpret_cast<int *>(lds + pad + 16);
    constexpr int RED_TILE = red_tile_ints(K, GROUP, MT);                    // ints per tile
    const int RED_OP = ((hdr->kind & PK_T_MASK) >> PK_T_SHIFT) * RED_TILE;   // ints per op slot

    // A wait that runs out only raises the LDS flag (the status word is
    // written once at the end): the stream waves then issue no global memory
    // operation besides their weight loads, so the compiler's wait counts
    // stay exact and each slot of the ring waits for its own loads only.
    auto report_timeout = [&]() {
        __hip_atomic_store(&abort_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };

    if (tid == 0) {
        img_cnt = 0;
        for (int q = 0; q < PG_SLOTS; ++q)
            sdone[q] = 0;
        isync = 0;
        abort_flag = 0;
    }
    for (int i = tid; i < PG_SLOTS * RED_OP; i += PG_THREADS)
        red0[i] = 0;
    if (tid < 4)
        reinterpret_cast<uint32_t *>(lds + pad)[tid] = 0u;
    __syncthreads();

    if (wave < PG_PREP) {
        // ===================== image waves =====================
        int phase = 0;
        auto img_sync = [&]() {   // barrier of the 4 image waves (LDS writes released)
            ++phase;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (lane == 0)
                __hip_atomic_fetch_add(&isync, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            wake_workgroup();
            if (!lds_wait_ge(&isync, PG_PREP * phase, &abort_flag) && lane == 0)
                report_timeout();
            asm volatile("" ::: "memory");
        };

        // ---- finish op j: y for this workgroup's rows of it
        auto finish = [&](int j) {
            const OpView op = op_view(ops_g, j);
            const int par = op.lpos % PG_SLOTS;
            int t0, ntl;
            my_tiles(op, t0, ntl);
            if (!lds_wait_ge(&sdone[par], PG_STREAM, &abort_flag) && lane == 0)
                report_timeout();
            asm volatile("" ::: "memory");
            int *red = red0 + par * RED_OP;
            const bool shared_y = WAITS && (op.flags & PF_Y_SHARED) != 0;
#pragma unroll
            for (int rr = 0; rr < PG_ROWS_PER_THREAD; ++rr) {
            const int lr = tid + rr * PG_PREP_THREADS;   // row of the workgroup's tiles
            if (rr > 0 && ntl * TILE_ROWS <= rr * PG_PREP_THREADS)
                break;
            const int row = t0 * TILE_ROWS + lr;
            const bool rowok = lr < ntl * TILE_ROWS && row < op.out;
            float yv[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m)
                yv[m] = 0.0f;
            if (GROUP && rowok) {
                // the stream waves' per-(tile, wave) slots, added in wave order
                const float *rf = reinterpret_cast<const float *>(red);
                const int tl = lr / TILE_ROWS, i = lr % TILE_ROWS;
                float acc = 0.0f;
#pragma unroll
                for (int w = 0; w < PG_STREAM; ++w)
                    acc += rf[(tl * PG_STREAM + w) * TILE_ROWS + i];
                yv[0] = __builtin_ldexpf(acc, -shs[par][0]);
            } else if (rowok) {
                const int tl = lr / TILE_ROWS, i = lr % TILE_ROWS;
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    double sx = 0.0;
#pragma unroll
                    for (int v = 0; v < PG_PREP; ++v)
                        sx += wsum[par][m][v];
                    float y = 0.0f;
#pragma unroll
                    for (int k = 0; k < (GROUP ? 1 : K); ++k) {
                        const int *rp = red + ((tl * K + k) * NC + NLIMB * m) * TILE_ROWS + i;
                        const double t = (double)rp[0] + 256.0 * (double)rp[TILE_ROWS] +
                                         65536.0 * (double)rp[2 * TILE_ROWS];
                        // one explicit fma per plane, as in the flat kernel
                        y = __builtin_fmaf(h2f(sc_lds[par][k][lr]), (float)(t * (2.0 / 128.0) - sx), y);
                    }
                    yv[m] = __builtin_ldexpf(y, -shs[par][m]);
                }
            }
            // token m's outputs follow token m - 1's (y is [MT][out], or [MT][out / 2])
            const bool silu = (op.flags & PF_SILU) != 0;
            const int ycount = silu ? op.out / 2 : op.out;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float y = yv[m];
                if (silu) {
                    // (gate, up) rows 2i, 2i + 1 sit on neighbouring threads (tiles start at even rows)
                    const float up = __shfl_down(y, 1, RBQ_WAVE);
                    if (rowok && (tid & 1) == 0) {
                        const uint16_t h = silu_mul_f16(y, up);
                        GLOBAL uint16_t *dst = op.y + (size_t)m * ycount + row / 2;
                        if (shared_y)
                            __hip_atomic_store(dst, h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        else
                            *dst = h;
                    }
                } else if (rowok) {
                    const uint16_t h = f2h(y);
                    GLOBAL uint16_t *dst = op.y + (size_t)m * ycount + row;
                    if (shared_y)
                        __hip_atomic_store(dst, h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    else
                        *dst = h;
                }
            }
            }
            img_sync();   // every partial sum of the op has been read
            for (int e = tid; e < ntl * RED_TILE; e += PG_PREP_THREADS)
                red[e] = 0;
            if (tid == 0)
                __hip_atomic_store(&sdone[par], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (WAITS && (op.flags & PF_SIGNAL)) {
                // this workgroup's rows of y are stored (device-coherent) before it counts
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                img_sync();
                if (tid == 0)
                    __hip_atomic_fetch_add(op_counter(counters, j, b & (PG_CSPLIT - 1)), 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            }
        };

        // ---- wait until every workgroup has finished op j
        auto wait_op = [&](int j) {
            if (tid == 0) {
                const uint64_t deadline = __builtin_amdgcn_s_memrealtime() + PG_WAIT_TICKS;
                for (;;) {
                    int tot = 0;
#pragma unroll
                    for (int c = 0; c < PG_CSPLIT; ++c)
                        tot += __hip_atomic_load(op_counter(counters, j, c), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
                    if (tot >= Gl)   // every workgroup of the op's group
                        break;
                    if (__hip_atomic_load(&abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) ||
                        __builtin_amdgcn_s_memrealtime() > deadline) {
                        report_timeout();
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            img_sync();
        };

        // ---- the loads of an op's image, issued one op ahead: x (thread t
        // owns half-words H = t + j * 256, 16 columns each; past the row end it
        // loads the last one, quantised with scale 0) and the scales of the row
        // the thread finishes.  x that an earlier op writes is loaded only after
        // the wait, with device-coherent loads.
        v4u xw[MT][XU][2];
        uint16_t a_bits[PG_ROWS_PER_THREAD][K];
        auto load_x = [&](const OpView &op) {
            const int nh = (op.in >> 5) * 2;
            const int xu = (op.nchunks * CHUNK_WORDS * 2 + PG_PREP_THREADS - 1) / PG_PREP_THREADS;
            const bool shared_x = WAITS && (op.flags & PF_X_SHARED) != 0;
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int j = 0; j < XU; ++j) {
                v4u (&xwj)[2] = xw[m][j];
                xwj[0] = xwj[1] = (v4u){0u, 0u, 0u, 0u};
                if (j < xu) {
                    const int Hh = min(tid + j * PG_PREP_THREADS, nh - 1);
                    GLOBAL const uint16_t *src = op.x + (size_t)m * op.in + 16 * Hh;
                    if (shared_x) {
                        GLOBAL const uint64_t *p = reinterpret_cast<GLOBAL const uint64_t *>(src);
                        uint64_t q[4];
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            q[c] = __hip_atomic_load(p + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        xwj[0] = (v4u){(uint32_t)q[0], (uint32_t)(q[0] >> 32), (uint32_t)q[1],
                                       (uint32_t)(q[1] >> 32)};
                        xwj[1] = (v4u){(uint32_t)q[2], (uint32_t)(q[2] >> 32), (uint32_t)q[3],
                                       (uint32_t)(q[3] >> 32)};
                    } else {
                        GLOBAL const v4u *xp = reinterpret_cast<GLOBAL const v4u *>(src);
                        xwj[0] = xp[0];
                        xwj[1] = xp[1];
                    }
                }
            }
        };
        auto load_scales = [&](const OpView &op) {
            if (GROUP)   // g128 scales travel with the weights, to the stream waves
                return;
            int t0, ntl;
            my_tiles(op, t0, ntl);
#pragma unroll
            for (int rr = 0; rr < PG_ROWS_PER_THREAD; ++rr) {
                const int lr = tid + rr * PG_PREP_THREADS;
                const int row = t0 * TILE_ROWS + lr;
                const bool rowok = lr < ntl * TILE_ROWS && row < op.out;
#pragma unroll
                for (int k = 0; k < (GROUP ? 1 : K); ++k)
                    a_bits[rr][k] = rowok ? op.scales[(size_t)k * op.out + row] : (uint16_t)0;
            }
        };

        // this wave's part of op i's image and sums is written: count it
        auto publish = [&]() {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (lane == 0)
                __hip_atomic_fetch_add(&img_cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            wake_workgroup();
        };
        // the op reads the same x as the group's op before it: that image (and
        // the sums that go with it) serve again; only the scales are its own
        auto reuse = [&](const OpView &op) {
            const int par = op.lpos % PG_SLOTS, prev = (op.lpos + PG_SLOTS - 1) % PG_SLOTS;
            if (GROUP) {
                for (int g = tid; g < PG_MAX_G; g += PG_PREP_THREADS)
                    gsum[par][g] = gsum[prev][g];
            } else {
#pragma unroll
                for (int rr = 0; rr < PG_ROWS_PER_THREAD; ++rr)
#pragma unroll
                    for (int k = 0; k < K; ++k)
                        sc_lds[par][k][tid + rr * PG_PREP_THREADS] = a_bits[rr][k];
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (lane == 0)
                    wsum[par][m][wave] = wsum[prev][m][wave];
                if (tid == 0)
                    shs[par][m] = shs[prev][m];
            }
            publish();
        };

        // ---- build op i's activation image from xw, a_bits into its buffer
        auto build = [&](int i, const OpView &op) {
            const int par = op.lpos % PG_SLOTS;
            const int nh = (op.in >> 5) * 2;                  // half-words of the row
            const int hpad = op.nchunks * CHUNK_WORDS * 2;    // with the padded words
            const int xu = (hpad + PG_PREP_THREADS - 1) / PG_PREP_THREADS;
            // maximum of |x| per token (fp16 bits without the sign order like magnitudes)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                v2u16 mx2 = (v2u16){0, 0};
#pragma unroll
                for (int j = 0; j < XU; ++j)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            mx2 = __builtin_elementwise_max(mx2,
                                                            __builtin_bit_cast(v2u16, xw[m][j][h][c] & 0x7FFF7FFFu));
                const uint32_t mw = wave_max_u32_dpp(max((uint32_t)mx2.x, (uint32_t)mx2.y));
                if (lane == 0)
                    wmax[par][m][wave] = mw;
            }
            if (!GROUP) {
#pragma unroll
                for (int rr = 0; rr < PG_ROWS_PER_THREAD; ++rr)
#pragma unroll
                    for (int k = 0; k < K; ++k)
                        sc_lds[par][k][tid + rr * PG_PREP_THREADS] = a_bits[rr][k];
            }
            img_sync();
            // image entry (word w, bit s): the columns 32w + 8kk + s, kk = 0..3,
            // at [chunk w/16][s][lane group (w/4)%4][limb column][4 (w%4) + kk];
            // token m's limbs are columns 3m .. 3m + 2.  fma(x, 2^sh, 1.5 2^23)
            // leaves 2^22 + q in the mantissa, v = q + 0x808080 lies in
            // [0, 2^24) and its bytes xor 0x80 are the limbs
            unsigned char *img = lds + op.img_off;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                uint32_t mx = 0;
#pragma unroll
                for (int v = 0; v < PG_PREP; ++v)
                    mx = max(mx, wmax[par][m][v]);
                // |x| < 2^E; q = round(x 2^sh), sh = 22 - E, |q| <= 2^22
                const int e = (int)(mx >> 10);
                const int sh = 22 - ((e == 0 ? 1 : e) - 14);
                int psum = 0;
#pragma unroll
                for (int j = 0; j < XU; ++j) {
                    const int H = tid + j * PG_PREP_THREADS;
                    if (GROUP)
                        psum = 0;
                    if (j < xu && H < hpad) {
                        const float scale = H < nh ? __builtin_ldexpf(1.0f, sh) : 0.0f;
                        const int w = H >> 1, eh = H & 1;
                        unsigned char *dst = img + (w / CHUNK_WORDS) * IMG_CHUNK + ((w >> 2) & 3) * (NC * 16) +
                                             NLIMB * m * 16 + (w & 3) * 4 + 2 * eh;
#pragma unroll
                        for (int s = 0; s < 8; ++s) {
                            const uint32_t u0 = xw[m][j][0][s >> 1], u1 = xw[m][j][1][s >> 1];
                            const uint16_t h0 = (s & 1) ? (uint16_t)(u0 >> 16) : (uint16_t)u0;
                            const uint16_t h1 = (s & 1) ? (uint16_t)(u1 >> 16) : (uint16_t)u1;
                            const uint32_t v0 =
                                __builtin_bit_cast(uint32_t, __builtin_fmaf(h2f(h0), scale, 12582912.0f)) - 0x4ABF7F80u;
                            const uint32_t v1 =
                                __builtin_bit_cast(uint32_t, __builtin_fmaf(h2f(h1), scale, 12582912.0f)) - 0x4ABF7F80u;
                            psum += (int)(v0 + v1) - 2 * 0x808080;
                            const uint32_t l01 = __builtin_amdgcn_perm(v1, v0, 0x05010400u) ^ 0x80808080u;
                            const uint32_t l2 = __builtin_amdgcn_perm(v1, v0, 0x0C0C0602u) ^ 0x8080u;
                            unsigned char *d = dst + s * (4 * NC * 16);
                            *reinterpret_cast<uint16_t *>(d) = (uint16_t)l01;
                            *reinterpret_cast<uint16_t *>(d + 16) = (uint16_t)(l01 >> 16);
                            *reinterpret_cast<uint16_t *>(d + 32) = (uint16_t)l2;
                        }
                    }
                    if (GROUP && j < xu) {
                        // the 8 half-words of a 128-column group sit in 8
                        // consecutive lanes; lane 8m + 7 adds them
                        int g = psum;
                        g = dpp_row_add_i32<RBQ_DPP_ROW_SHR(1)>(g);
                        g = dpp_row_add_i32<RBQ_DPP_ROW_SHR(2)>(g);
                        g = dpp_row_add_i32<RBQ_DPP_ROW_SHR(4)>(g);
                        if ((lane & 7) == 7 && H < hpad)
                            gsum[par][H >> 3] = g;
                    }
                }
                if (!GROUP) {
                    const double ws = wave_sum_f64_dpp((double)psum);   // sum of q over the wave's columns (exact)
                    if (lane == 0)
                        wsum[par][m][wave] = ws;
                }
                if (tid == 0)
                    shs[par][m] = sh;
            }
            publish();
        };

        // this workgroup runs the ops of its group, in list order
        auto next_mine = [&](int i) {
            while (i < n_ops && op_view(ops_g, i).grp != mygrp)
                ++i;
            return i;
        };
        // the group's ops are linked (each descriptor names the group's next
        // op), so only the first one is searched for
        auto finish_upto = [&](int &next_fin, int upto) {
            while (next_fin <= upto) {
                const int nf = op_view(ops_g, next_fin).next;
                finish(next_fin);
                next_fin = nf;
            }
        };
        int i = next_mine(0);
        int next_fin = i;
        OpView cur = op_view(ops_g, i < n_ops ? i : 0);
        if (i < n_ops) {
            if (!(WAITS && (cur.flags & PF_X_SHARED)))
                load_x(cur);
            load_scales(cur);
        }
        while (i < n_ops) {
            // finish what the op waits for, the op whose slot of partial sums
            // and scales it takes, and the last op whose image shares LDS
            // bytes with its own
            finish_upto(next_fin, max(WAITS ? cur.wait_for : -1, cur.free_after));
            if (WAITS && cur.wait_for >= 0)
                wait_op(cur.wait_for);
            if (cur.flags & PF_REUSE) {
                reuse(cur);
            } else {
                if (WAITS && (cur.flags & PF_X_SHARED))
                    load_x(cur);
                build(i, cur);
            }
            const int nx = cur.next;
            if (nx < n_ops) {
                // the next op's loads go out now, to arrive while this op streams
                cur = op_view(ops_g, nx);
                if (!(cur.flags & ((WAITS ? PF_X_SHARED : 0u) | PF_REUSE)))
                    load_x(cur);
                load_scales(cur);
            }
            i = nx;
        }
        finish_upto(next_fin, n_ops - 1);
    } else {
        // ===================== stream waves =====================
        const int sw = wave - PG_PREP;
        const int total = wave_units[b * PG_STREAM + sw];

        // ---- load cursor: the next (op, unit) whose weights are requested
        int lop = 0, lnext = 0, lu = 0, lu1 = 0, lt0 = 0, lnch = 1, lwords = 4, lout = 1;
        bool ltiles = false;
        uint32_t lmagic = 0;
        const OpView op0 = op_view(ops_g, 0);
        GLOBAL const uint32_t *lplanes = op0.planes;
        GLOBAL const uint16_t *lscales = op0.scales;   // g128: the op's scale tiles
        size_t lstride = 0;
        auto lseek = [&]() {   // the first op from lop on that gives this wave units
            while (lop < n_ops) {
                const OpView op = op_view(ops_g, lop);
                int t0, ntl;
                my_tiles(op, t0, ntl);
                op_units(ntl * op.nchunks, op.wrot, sw, lu, lu1);
                if (lu < lu1) {
                    lt0 = t0;
                    lnch = op.nchunks;
                    lwords = op.in >> 5;
                    lout = op.out;
                    lplanes = op.planes;
                    lscales = op.scales;
                    ltiles = TILES || (op.flags & PF_TILES) != 0;
                    // words per plane: the tile layout pads rows and words to whole units
                    lstride = ltiles ? (size_t)((op.out + TILE_ROWS - 1) / TILE_ROWS) * op.nchunks * 256
                                     : (size_t)op.out * lwords;
                    lmagic = op.magic;
                    lnext = op.next;
                    return;
                }
                lop = op.grp == mygrp ? op.next : lop + 1;
            }
        };
        // lanes (li, lg) read words 4lg .. 4lg+3 of row li of a unit's tile
        // (in the tile layout: bytes 16 lane .. 16 lane + 15 of the unit's
        // block); past the last unit the last address is loaded again (a wave
        // with no units at all reads the first words of op 0)
        GLOBAL const uint32_t *lastp = lplanes + min(4 * lg, (op0.in >> 5) - 4);
        size_t laststride = (size_t)op0.out * (op0.in >> 5);
        // g128 (tile layouts only): lane (li, lg) loads, per pair of planes, the
        // 16 bytes with the scales of rows 4lg .. 4lg+3 of the unit's group
        // min(li / 3, 3) (the MFMA column li = 3 group + limb it holds)
        constexpr int KS = GROUP ? K / 2 : 0;
        constexpr int KR = K + KS;
        const int sc_lane = (min(li / 3, 3) * 4 + lg) * 8;
        GLOBAL const uint16_t *lastsp = lscales + sc_lane;
        lseek();
        auto load_next = [&](v4u (&slot)[KR]) {
            if (lop < n_ops) {
                const int tq = (int)(((uint32_t)lu * lmagic) >> 21);
                if (TILES || ltiles) {
                    const size_t unit = (size_t)(lt0 + tq) * lnch + (lu - tq * lnch);
                    lastp = lplanes + unit * 256 + 4 * lane;
                    if (GROUP)
                        lastsp = lscales + unit * (K * 64) + sc_lane;
                } else {
                    const int row = min((lt0 + tq) * TILE_ROWS + li, lout - 1);
                    const int wi = min((lu - tq * lnch) * CHUNK_WORDS + 4 * lg, lwords - 4);
                    lastp = lplanes + (size_t)row * lwords + wi;
                }
                laststride = lstride;
                if (++lu == lu1) {
                    lop = lnext;
                    lseek();
                }
            }
            // Every plane and scale byte is read once per run.  On the tile
            // layout (a wave load is one whole 1 KB block) the loads are
            // non-temporal: the Llama-2-7B step took 280 us instead of 295 us.
            // On the row layout a 128-byte line holds the half-lines of two
            // units, and kept in L2 the second half is a hit (non-temporal
            // there: 398 us instead of 320 us).
#pragma unroll
            for (int k = 0; k < K; ++k) {
                GLOBAL const v4u *src = reinterpret_cast<GLOBAL const v4u *>(lastp + k * laststride);
                if constexpr (TILES)
                    slot[k] = __builtin_nontemporal_load(src);
                else
                    slot[k] = *src;
            }
#pragma unroll
            for (int pp = 0; pp < KS; ++pp) {
                GLOBAL const v4u *src = reinterpret_cast<GLOBAL const v4u *>(lastsp + pp * 128);
                if constexpr (TILES)
                    slot[K + pp] = __builtin_nontemporal_load(src);
                else
                    slot[K + pp] = *src;
            }
        };

        // ---- consume cursor: the op and unit the MFMAs work on
        int cop = 0, cnext = 0, cu = 0, cu1 = 0, cnch = 1, ctile = 0, cchunk = 0, cimg = 0, cpar = 0;
        auto report = [&](int par) {   // this wave is done with the op in slot par
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (lane == 0)
                __hip_atomic_fetch_add(&sdone[par], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            wake_workgroup();
        };
        // wait for op cop's image; skip another group's ops, and report this
        // group's ops without units here
        auto cseek = [&]() {
            while (cop < n_ops) {
                const OpView op = op_view(ops_g, cop);
                if (op.grp == mygrp) {
                    if (!lds_wait_ge(&img_cnt, PG_PREP * (op.lpos + 1), &abort_flag) && lane == 0)
                        report_timeout();
                    asm volatile("" ::: "memory");
                    int t0, ntl;
                    my_tiles(op, t0, ntl);
                    op_units(ntl * op.nchunks, op.wrot, sw, cu, cu1);
                    cpar = op.lpos % PG_SLOTS;
                    if (cu < cu1) {
                        cnch = op.nchunks;
                        cimg = op.img_off;
                        const int tq = (int)(((uint32_t)cu * op.magic) >> 21);
                        ctile = tq;
                        cchunk = cu - tq * cnch;
                        cnext = op.next;
                        return;
                    }
                    report(cpar);
                }
                cop = op.grp == mygrp ? op.next : cop + 1;
            }
        };

        // per-row ops: running int32 totals per plane and bit position
        v4i acc[GROUP ? 1 : K][8];
        uint32_t tprev[GROUP ? 1 : K][4];
#pragma unroll
        for (int k = 0; k < (GROUP ? 1 : K); ++k) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[k][j] = (v4i){0, 0, 0, 0};
#pragma unroll
            for (int v = 0; v < 4; ++v)
                tprev[k][v] = 0u;
        }
        // g128 ops: MFMA column li = 3t + l is limb l of the chunk's group t,
        // fed only from lane group t (the B operand is zero elsewhere), so
        // C[i][li] is row i's sum over group t alone; the lanes apply the
        // group's scales and keep fp32 running sums yv of rows 4lg .. 4lg+3
        // (times 2^-(8l+1); cl restores it at the flush, where the 16 columns
        // of each row are added).  2 S - sum q = sum_l 2^(8l+1) (T_l - [l=0] sum q / 2).
        const bool g_live = li < 3 * 4;
        const bool g_b = g_live && li / 3 == lg;
        const int g_t = min(li / 3, 3);
        const float g_zq = (g_live && li % 3 == 0) ? -0.5f : 0.0f;
        const float g_cl = g_live ? __builtin_ldexpf(1.0f, 8 * (li % 3) + 1) : 0.0f;
        float yv[4] = {0.0f, 0.0f, 0.0f, 0.0f};

        v4u ring[RING][KR];
#pragma unroll
        for (int d = 0; d < RING; ++d)
            load_next(ring[d]);
        cseek();

        auto consume = [&](const v4u (&wv)[KR]) {
            const int par = cpar;
            if constexpr (GROUP) {
                ++cu;
                const bool tile_end = cchunk + 1 == cnch;
                const bool op_end = cu == cu1;
                const unsigned char *bp = g_b ? lds + cimg + (lg * NC + li - 3 * lg) * 16 + cchunk * IMG_CHUNK
                                              : lds + pad;
                const int bstride = g_b ? 4 * NC * 16 : 0;
                v4i ga[K];
#pragma unroll
                for (int k = 0; k < K; ++k)
                    ga[k] = (v4i){0, 0, 0, 0};
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const v4i bv = *reinterpret_cast<const v4i *>(bp + s * bstride);
#pragma unroll
                    for (int k = 0; k < K; ++k) {
                        const v4i av = (v4i){(int)((wv[k].x >> s) & 0x01010101u), (int)((wv[k].y >> s) & 0x01010101u),
                                             (int)((wv[k].z >> s) & 0x01010101u), (int)((wv[k].w >> s) & 0x01010101u)};
                        ga[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, ga[k], 0, 0, 0);
                    }
                }
                // The results of the last MFMAs are read next.  With only the
                // compiler's wait states between the last MFMA and the first
                // read, that read returned a stale first result register now
                // and then (rows 4q of a tile wrong, differently from run to
                // run); 16 more wait states here, tied to the result registers.
                if constexpr (K == 2)
                    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(ga[0]), "+v"(ga[1]));
                else
                    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(ga[0]), "+v"(ga[1]), "+v"(ga[2]), "+v"(ga[3]));
                const float gq = (float)gsum[par][cchunk * 4 + g_t];
#pragma unroll
                for (int k = 0; k < K; ++k)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const uint32_t hw = wv[K + k / 2][(k & 1) * 2 + (v >> 1)];
                        const float a = h2f((uint16_t)(hw >> (16 * (v & 1))));
                        yv[v] = __builtin_fmaf(a, __builtin_fmaf(g_zq, gq, (float)ga[k][v]), yv[v]);
                    }
                if (tile_end || op_end) {
                    float *rf = reinterpret_cast<float *>(red0 + par * RED_OP) + (ctile * PG_STREAM + sw) * TILE_ROWS;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        float x = yv[v] * g_cl;
                        x = dpp_row_add_f32<RBQ_DPP_ROW_SHR(1)>(x);
                        x = dpp_row_add_f32<RBQ_DPP_ROW_SHR(2)>(x);
                        x = dpp_row_add_f32<RBQ_DPP_ROW_SHR(4)>(x);
                        x = dpp_row_add_f32<RBQ_DPP_ROW_SHR(8)>(x);
                        if (li == 15)
                            rf[4 * lg + v] = x;
                        yv[v] = 0.0f;
                    }
                }
                // next chunk (as selects: written as two branches, the compiler
                // merged them into one increment through a pointer to either
                // variable, which put both on the stack)
                ctile += tile_end ? 1 : 0;
                cchunk = tile_end ? 0 : cchunk + 1;
                if (op_end) {
                    report(cpar);
                    cop = cnext;
                    cseek();
                }
            } else {
                const unsigned char *bp = li < NC ? lds + cimg + (lg * NC + li) * 16 + cchunk * IMG_CHUNK
                                                  : lds + pad;
                const int bstride = li < NC ? 4 * NC * 16 : 0;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const v4i bv = *reinterpret_cast<const v4i *>(bp + s * bstride);
                    const uint32_t mask = 0x01010101u << s;
#pragma unroll
                    for (int k = 0; k < K; ++k) {
                        const v4i av = (v4i){(int)(wv[k].x & mask), (int)(wv[k].y & mask), (int)(wv[k].z & mask),
                                             (int)(wv[k].w & mask)};
                        acc[k][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc[k][s], 0, 0, 0);
                    }
                }
                // next chunk; at a tile's end or the wave's last unit of the op, add
                // T = sum_{s<7} 2^(7-s) acc_s - acc_7 = 2^7 sum(bit * limb) into LDS
                ++cu;
                const bool tile_end = ++cchunk == cnch;
                const bool op_end = cu == cu1;
                if (tile_end || op_end) {
                    // (the empty asm keeps the recombination below inside this
                    // branch: hoisted, it cost ~80 VALU operations on every unit)
#pragma unroll
                    for (int k = 0; k < K; ++k)
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            asm volatile("" : "+v"(acc[k][j]));
                    // The accumulators are never cleared: T is linear in them, so
                    // the tile's share is T now less T at the previous flush, all
                    // modulo 2^32 (the int32 sums wrap; the share stays below
                    // 2^29).  That saves clearing 64 registers per flush.
                    int *rp = red0 + par * RED_OP + ctile * K * NC * TILE_ROWS + li * TILE_ROWS + 4 * lg;
#pragma unroll
                    for (int k = 0; k < K; ++k)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            uint32_t t = (uint32_t)acc[k][0][v];
#pragma unroll
                            for (int q = 1; q < 7; ++q)
                                t = (t << 1) + (uint32_t)acc[k][q][v];
                            t = (t << 1) - (uint32_t)acc[k][7][v];
                            const uint32_t share = t - tprev[k][v];
                            tprev[k][v] = t;
                            if (li < NC)
                                __hip_atomic_fetch_add(rp + k * NC * TILE_ROWS + v, (int)share, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_WORKGROUP);
                        }
                }
                if (tile_end) {
                    cchunk = 0;
                    ++ctile;
                }
                if (op_end) {
                    report(cpar);
                    cop = cnext;
                    cseek();
                }
            }
        };

        const int nbk = (total + RING - 1) / RING;
        for (int bi = 0; bi + 1 < nbk; ++bi) {
#pragma unroll
            for (int d = 0; d < RING; ++d) {
                consume(ring[d]);
                load_next(ring[d]);
            }
        }
        if (nbk > 0) {
#pragma unroll
            for (int d = 0; d < RING; ++d)
                if ((nbk - 1) * RING + d < total)
                    consume(ring[d]);
        }
        // ops after this wave's last unit that give it none are reported by
        // cseek (also when the wave has no units at all)
    }
    __syncthreads();

    if (tid == 0 && status != nullptr && abort_flag)
        __hip_atomic_fetch_or(status, (int)RBQ_STATUS_PROGRAM_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the last workgroup to finish clears the op counters for the next run
    int *done_counter = op_counter(counters, n_ops, 0);
    if (tid == 0) {
        const int done = __hip_atomic_fetch_add(done_counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh.last_wg = done == G - 1;
    }
    __syncthreads();
    if (sh.last_wg) {
        for (int e = tid; e < n_ops * PG_CSPLIT; e += PG_THREADS)
            __hip_atomic_store(op_counter(counters, e / PG_CSPLIT, e % PG_CSPLIT), 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        if (tid == 0)
            __hip_atomic_store(done_counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

uint32_t image_checksum(const unsigned char *img, size_t bytes) {
    // FNV-1a over everything after the header's checksum field
    uint32_t h = 2166136261u;
    for (size_t i = 0; i < bytes; ++i) {
        if (i >= offsetof(ProgHeader, checksum) && i < offsetof(ProgHeader, checksum) + 4)
            continue;
        h ^= img[i];
        h *= 16777619u;
    }
    return h;
}

bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

}  // namespace

size_t program_bytes(int n_ops) {
    if (n_ops < 1 || n_ops > RBQ_PROGRAM_MAX_OPS)
        return 0;
    return image_bytes(n_ops, program_num_cus());
}

rbq_status program_build(const rbq_program_op *ops, int n_ops, int K, void *image, size_t bytes) {
    if (ops == nullptr || image == nullptr || n_ops < 1 || n_ops > RBQ_PROGRAM_MAX_OPS || K < 1 || K > 8)
        return n_ops > RBQ_PROGRAM_MAX_OPS ? RBQ_ERR_UNSUPPORTED : RBQ_ERR_INVALID_ARG;
    // a program is of per-row ops (K <= 2) or of g128 ops (K = 2 or 4) alone
    if (ops[0].group_size != 0 && ops[0].group_size != 128)
        return RBQ_ERR_INVALID_ARG;
    const bool group = ops[0].group_size == 128;
    if (group ? (K != 2 && K != 4) : K > 2)
        return RBQ_ERR_UNSUPPORTED;
    // tokens per op: 0 and 1 both mean one; ops of 2 or 4 tokens are per-row
    // K = 2 ops on the tile layout in programs without waits, every op of
    // the program with the same count
    if (ops[0].tokens < 0)
        return RBQ_ERR_INVALID_ARG;
    const int tok = ops[0].tokens <= 1 ? 1 : ops[0].tokens;
    if (tok != 1 && tok != 2 && tok != 4)
        return RBQ_ERR_UNSUPPORTED;
    if (tok > 1 && (group || K != 2))
        return RBQ_ERR_UNSUPPORTED;
    const int G = program_num_cus();
    if (G > 4095)   // the tile split keeps tiles % G in 12 bits
        return RBQ_ERR_UNSUPPORTED;
    if (bytes < image_bytes(n_ops, G))
        return RBQ_ERR_INVALID_ARG;
    auto al = [](const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; };
    const int max_out = PG_MAX_TILES * TILE_ROWS * G;
    std::vector<size_t> xb(n_ops), yb(n_ops), pb(n_ops), sb(n_ops);
    for (int i = 0; i < n_ops; ++i) {
        const rbq_program_op &o = ops[i];
        if (o.planes == nullptr || o.scales == nullptr || o.x == nullptr || o.y == nullptr)
            return RBQ_ERR_INVALID_ARG;
        if (o.tokens < 0 || (o.tokens <= 1 ? 1 : o.tokens) != tok)
            return RBQ_ERR_INVALID_ARG;
        if (tok > 1 && (o.planes_layout != RBQ_LAYOUT_TILES || o.wait_for >= 0 || o.in_features > max_in_of(tok)))
            return RBQ_ERR_UNSUPPORTED;
        if (o.out_features < 1 || o.in_features < 1 || o.in_features % 32 != 0)
            return RBQ_ERR_INVALID_ARG;
        if (o.epilogue != RBQ_EPILOGUE_NONE && o.epilogue != RBQ_EPILOGUE_SILU_MUL)
            return RBQ_ERR_INVALID_ARG;
        if (o.epilogue == RBQ_EPILOGUE_SILU_MUL && o.out_features % 2 != 0)
            return RBQ_ERR_INVALID_ARG;
        if (o.wait_for < -1 || o.wait_for >= i)
            return RBQ_ERR_INVALID_ARG;
        if (o.planes_layout != RBQ_LAYOUT_ROWS && o.planes_layout != RBQ_LAYOUT_TILES)
            return RBQ_ERR_INVALID_ARG;
        if (o.group_size != 0 && o.group_size != 128)
            return RBQ_ERR_INVALID_ARG;
        if ((o.group_size == 128) != group || (group && o.planes_layout != RBQ_LAYOUT_TILES))
            return RBQ_ERR_UNSUPPORTED;
        if (o.in_features % 128 != 0 || o.in_features > PG_MAX_CHUNKS * CHUNK_WORDS * 32 ||
            o.out_features > max_out)
            return RBQ_ERR_UNSUPPORTED;
        if (!al(o.planes, 16) || !al(o.x, 16) || !al(o.scales, group ? 16 : 2) || !al(o.y, 2))
            return RBQ_ERR_ALIGNMENT;
        xb[i] = (size_t)tok * o.in_features * 2;
        yb[i] = (size_t)tok * (o.epilogue == RBQ_EPILOGUE_SILU_MUL ? o.out_features / 2 : o.out_features) * 2;
        pb[i] = o.planes_layout == RBQ_LAYOUT_TILES ? tiles_bytes(K, o.out_features, o.in_features)
                                                    : (size_t)K * o.out_features * (o.in_features / 32) * 4;
        sb[i] = group ? scale_tiles_bytes(K, o.out_features, o.in_features) : (size_t)K * o.out_features * 2;
    }
    // Ordering.  Workgroups run the ops in order, each on its own rows, so two
    // accesses of ops j < i to one buffer are ordered across workgroups only
    // when some op in (j, i] waits for an op >= j.  y must not overlap its own
    // x or any weights.
    std::vector<uint32_t> flags(n_ops, 0u);
    for (int i = 0; i < n_ops; ++i) {
        if (ops[i].epilogue == RBQ_EPILOGUE_SILU_MUL)
            flags[i] |= PF_SILU;
        if (ops[i].planes_layout == RBQ_LAYOUT_TILES)
            flags[i] |= PF_TILES;
        if (ops[i].wait_for >= 0)
            flags[ops[i].wait_for] |= PF_SIGNAL;
        if (ranges_overlap(ops[i].y, yb[i], ops[i].x, xb[i]))
            return RBQ_ERR_INVALID_ARG;
        for (int j = 0; j < n_ops; ++j)
            if (ranges_overlap(ops[i].y, yb[i], ops[j].planes, pb[j]) ||
                ranges_overlap(ops[i].y, yb[i], ops[j].scales, sb[j]))
                return RBQ_ERR_INVALID_ARG;
        int m = -1;   // max wait_for over ops j+1 .. i
        for (int j = i - 1; j >= 0; --j) {
            m = std::max(m, ops[j + 1].wait_for);
            const bool raw = ranges_overlap(ops[i].x, xb[i], ops[j].y, yb[j]);
            const bool war = ranges_overlap(ops[i].y, yb[i], ops[j].x, xb[j]);
            const bool waw = ranges_overlap(ops[i].y, yb[i], ops[j].y, yb[j]);
            if ((raw || war || waw) && m < j)
                return RBQ_ERR_INVALID_ARG;
            if (raw) {
                flags[i] |= PF_X_SHARED;
                flags[j] |= PF_Y_SHARED;
            }
            if (war || waw)
                flags[i] |= PF_Y_SHARED;
        }
    }
    unsigned char *img = static_cast<unsigned char *>(image);
    memset(img, 0, image_bytes(n_ops, G));
    ProgHeader *h = reinterpret_cast<ProgHeader *>(img);
    ProgOp *d = reinterpret_cast<ProgOp *>(h + 1);
    int32_t *wu = reinterpret_cast<int32_t *>(d + n_ops);
    int max_img = 0;
    for (int i = 0; i < n_ops; ++i)
        max_img = std::max(max_img, ((ops[i].in_features / 32 + CHUNK_WORDS - 1) / CHUNK_WORDS) * img_chunk_bytes(tok));
    const size_t budget = program_dynamic_lds(K, group, tok);
    // LDS the partial sums take when each workgroup gets up to mt tiles of an op
    auto fixed_lds = [&](int mt) { return 16 + (size_t)PG_SLOTS * mt * red_tile_ints(K, group, tok) * 4; };
    auto max_tiles_of = [&](int gl) {
        int mt = 1;
        for (int i = 0; i < n_ops; ++i)
            mt = std::max(mt, ((ops[i].out_features + TILE_ROWS - 1) / TILE_ROWS + gl - 1) / gl);
        return mt;
    };
    // Op groups.  Without waits the ops are independent, and the workgroups
    // are split into P groups of G / P: each op goes to one group (below:
    // balanced by plane bytes), whose workgroups take its tiles,
    // so every workgroup runs 1/P of the ops with P times their tiles each.
    // What a workgroup spends per op (images, finishes, flushes, cursors) is
    // then spread over P times the units.  The most groups whose largest op
    // fits a workgroup (PG_MAX_TILES tiles, and its partial sums in LDS next
    // to the largest image) are taken.  Programs with waits keep one group:
    // their ops run one after another anyway.
    int P = 1;
    {
        bool waits = false;
        for (int i = 0; i < n_ops; ++i)
            waits |= ops[i].wait_for >= 0;
        // (ops of several tokens: the most groups that leave room for two of
        // the largest images, so that the next op's image is built while an
        // op streams; failing that, the most that fit one)
        auto fits = [&](int cand, int images) {
            return !waits && n_ops >= cand && G % cand == 0 && max_tiles_of(G / cand) <= PG_MAX_TILES &&
                   fixed_lds(max_tiles_of(G / cand)) + (size_t)images * max_img <= budget;
        };
        int cand = RBQ_PROGRAM_GROUPS;
        if (tok > 1)
            while (cand > 1 && !fits(cand, 2))
                cand /= 2;
        if (tok == 1 || !fits(cand, 2)) {
            cand = RBQ_PROGRAM_GROUPS;
            while (cand > 1 && !fits(cand, 1))
                cand /= 2;
        }
        P = cand;
    }
    const int max_tiles = max_tiles_of(G / P);
    // LDS: the image arena takes what the partial sums leave
    const size_t fixed = fixed_lds(max_tiles);
    if (max_tiles > PG_MAX_TILES || fixed + (size_t)max_img > budget)
        return RBQ_ERR_UNSUPPORTED;
    const int arena = (int)((budget - fixed) / 16 * 16);
    const int Gl = G / P;
    std::vector<int> grp(n_ops, 0);
    {
        // largest op first, each to the group with the fewest bytes so far;
        // a group then runs its ops in program order.  (Taken in program
        // order instead, the Llama-2-7B step left its heaviest group 6 % above
        // the mean, and the step waits for that group.)
        std::vector<int> order(n_ops);
        for (int i = 0; i < n_ops; ++i)
            order[i] = i;
        std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
            return (double)pb[a] + (double)sb[a] > (double)pb[b] + (double)sb[b];
        });
        std::vector<double> load(P, 0.0);
        for (const int i : order) {
            int g = 0;
            for (int q = 1; q < P; ++q)
                if (load[q] < load[g])
                    g = q;
            grp[i] = g;
            load[g] += (double)pb[i] + (double)sb[i];
        }
    }
    // Per group: images go into the arena one after another, wrapping to 0
    // when one would pass its end; an op is built only once every earlier op
    // of its group whose image shares bytes with its own is finished, and the
    // op PG_SLOTS places back in the group, whose slot it takes (free_after).
    struct Placed { int op, lo, hi; };
    struct GroupPlan {
        std::vector<Placed> live;   // images placed so far, oldest first, with their byte ranges
        std::vector<int> seq;       // the group's ops so far
        int trot = 0, wrot = 0, next_off = 0, prev_off = 0;
        int last_trot = 0;          // the tile rotation of the group's op before
    };
    std::vector<GroupPlan> gp(P);
    for (int i = 0; i < n_ops; ++i) {
        const rbq_program_op &o = ops[i];
        GroupPlan &g = gp[grp[i]];
        ProgOp &p = d[i];
        p.planes = o.planes;
        p.scales = o.scales;
        p.x = o.x;
        p.y = o.y;
        p.out = o.out_features;
        p.in = o.in_features;
        p.wait_for = (int16_t)o.wait_for;
        p.flags = flags[i] | ((uint32_t)grp[i] << PF_GRP_SHIFT);
        const int tiles = (o.out_features + TILE_ROWS - 1) / TILE_ROWS;
        const int base = tiles / Gl, extra = tiles % Gl;
        p.split = (uint32_t)base | ((uint32_t)extra << 8) | (PG_NO_NEXT << 20);
        const int nch = (o.in_features / 32 + CHUNK_WORDS - 1) / CHUNK_WORDS;
        p.magic = ((1u << 21) + nch - 1) / nch;
        const int lpos = (int)g.seq.size();
        // an op on the planes of the group's op before (another batch of
        // tokens) takes that op's tiles: each workgroup re-reads the planes it
        // has just read, from its L2
        const bool same_planes = !g.seq.empty() && ops[g.seq.back()].planes == o.planes &&
                                 ops[g.seq.back()].out_features == o.out_features;
        const int trot_op = same_planes ? g.last_trot : g.trot;
        p.trot = trot_op | (lpos << 16);
        if (!g.seq.empty())   // link the group's previous op to this one
            d[g.seq.back()].split = (d[g.seq.back()].split & 0xFFFFFu) | ((uint32_t)i << 20);
        // an op that reads the same x as the group's op before it (and no op
        // writes it) takes that op's image
        const int prev = g.seq.empty() ? -1 : g.seq.back();
        const bool same = prev >= 0 && o.x == ops[prev].x && o.in_features == ops[prev].in_features &&
                          !(flags[i] & PF_X_SHARED) && !(flags[prev] & PF_X_SHARED);
        int fa = lpos >= PG_SLOTS ? g.seq[lpos - PG_SLOTS] : -1;
        int off;
        if (same) {
            p.flags |= PF_REUSE;
            off = g.prev_off;
            g.live.back().op = i;   // the image is in use until this op
        } else {
            const int size = nch * img_chunk_bytes(tok);
            off = g.next_off + size <= arena ? g.next_off : 0;
            for (const Placed &q : g.live)
                if (q.lo < off + size && off < q.hi)
                    fa = std::max(fa, q.op);
            g.live.push_back({i, off, off + size});
            g.next_off = off + size;
        }
        p.free_after = (int16_t)fa;
        g.prev_off = off;
        g.seq.push_back(i);
        p.nch_img = (uint32_t)nch | ((uint32_t)(off / 16) << 8);
        p.flags |= (uint32_t)g.wrot << PF_WROT_SHIFT;
        if (!same_planes) {
            g.last_trot = g.trot;
            g.trot = (g.trot + extra) % Gl;
        }
        g.wrot = (g.wrot + ((tiles + Gl - 1) / Gl) * nch) % PG_STREAM;
        for (int bl = 0; bl < Gl; ++bl) {
            const int bb = grp[i] * Gl + bl;
            int t0, ntl;
            op_tiles(base, extra, trot_op, bl, Gl, t0, ntl);
            for (int sw = 0; sw < PG_STREAM; ++sw) {
                int u0, u1;
                op_units(ntl * nch, (int)((p.flags >> PF_WROT_SHIFT) & 15u), sw, u0, u1);
                wu[bb * PG_STREAM + sw] += u1 - u0;
            }
        }
    }
    // Each MFMA adds at most 64 * 128 * 128 = 2^20 in magnitude to an int32
    // accumulator, and the stream waves never clear theirs during a run: up
    // to 2^11 units per wave keeps every sum below 2^31.
    for (int q = 0; q < G * PG_STREAM; ++q)
        if (wu[q] >= (1 << 11))
            return RBQ_ERR_UNSUPPORTED;
    const size_t lds = std::max(PG_MIN_LDS, fixed + (size_t)arena);
    h->magic = PG_MAGIC;
    h->n_ops = n_ops;
    h->K = K;
    h->grid = G;
    h->lds_bytes = (uint32_t)lds;
    h->arena_bytes = arena;
    h->kind = PK_TILES | (group ? PK_GROUP : 0) | (P << PK_P_SHIFT) | (max_tiles << PK_T_SHIFT) |
              ((tok == 4 ? 2 : tok == 2 ? 1 : 0) << PK_MT_SHIFT);
    for (int i = 0; i < n_ops; ++i) {
        h->kind |= ops[i].wait_for >= 0 ? PK_WAITS : 0;
        h->kind &= ops[i].planes_layout == RBQ_LAYOUT_TILES ? ~0 : ~PK_TILES;
    }
    h->checksum = image_checksum(img, image_bytes(n_ops, G));
    return RBQ_OK;
}

#ifndef RBQ_PROGRAM_RING
#define RBQ_PROGRAM_RING 2
#endif

rbq_status program_check(const void *image) {
    const ProgHeader *h = static_cast<const ProgHeader *>(image);
    if (h == nullptr || h->magic != PG_MAGIC || h->n_ops < 1 || h->n_ops > RBQ_PROGRAM_MAX_OPS ||
        h->grid != program_num_cus() ||
        (h->kind & ~(PK_WAITS | PK_TILES | PK_GROUP | PK_P_MASK | PK_T_MASK | PK_MT_MASK)) != 0)
        return RBQ_ERR_INVALID_ARG;
    const int mt = (h->kind & PK_T_MASK) >> PK_T_SHIFT;
    if (mt < 1 || mt > PG_MAX_TILES)
        return RBQ_ERR_INVALID_ARG;
    const int P = (h->kind & PK_P_MASK) >> PK_P_SHIFT;
    if ((P != 1 && P != 2 && P != 4 && P != 8) || h->grid % P != 0 || (P > 1 && (h->kind & PK_WAITS)))
        return RBQ_ERR_INVALID_ARG;
    const bool group = (h->kind & PK_GROUP) != 0;
    if (group ? (h->K != 2 && h->K != 4) || !(h->kind & PK_TILES) : (h->K != 1 && h->K != 2))
        return RBQ_ERR_INVALID_ARG;
    const int lmt = (h->kind & PK_MT_MASK) >> PK_MT_SHIFT;   // log2 of the tokens per op
    if (lmt > 2 || (lmt > 0 && (group || h->K != 2 || !(h->kind & PK_TILES) || (h->kind & PK_WAITS))))
        return RBQ_ERR_INVALID_ARG;
    if (image_checksum(static_cast<const unsigned char *>(image), image_bytes(h->n_ops, h->grid)) != h->checksum)
        return RBQ_ERR_INVALID_ARG;
    // never launch a layout that would not fit the compute unit's LDS
    if ((size_t)h->lds_bytes > program_dynamic_lds(h->K, group, 1 << lmt))
        return RBQ_ERR_UNSUPPORTED;
    return RBQ_OK;
}

int program_num_ops(const void *image) { return static_cast<const ProgHeader *>(image)->n_ops; }

size_t program_counters_bytes(int n_ops) { return program_counter_ints(n_ops) * sizeof(int32_t); }

hipError_t launch_program(const void *image, const void *image_dev, int32_t *counters, int32_t *status,
                          hipStream_t st) {
    const ProgHeader *h = static_cast<const ProgHeader *>(image);
    const ProgHeader *hd = static_cast<const ProgHeader *>(image_dev);
    // programs without waits take the kernel with the waiting code compiled
    // out, programs of tiled ops only the one without row addressing
#define RBQ_LAUNCH_PROGRAM(KK, WW, TT, GG)                                                                  \
    hipLaunchKernelGGL((gemv_program_kernel<KK, RBQ_PROGRAM_RING, WW, TT, GG>), dim3(h->grid), dim3(PG_THREADS), \
                       h->lds_bytes, st, hd, h->n_ops, h->checksum, counters, status)
#define RBQ_LAUNCH_PROGRAM_K(KK)                                         \
    switch (h->kind & (PK_WAITS | PK_TILES)) {                           \
    case 0: RBQ_LAUNCH_PROGRAM(KK, false, false, false); break;          \
    case PK_WAITS: RBQ_LAUNCH_PROGRAM(KK, true, false, false); break;    \
    case PK_TILES: RBQ_LAUNCH_PROGRAM(KK, false, true, false); break;    \
    default: RBQ_LAUNCH_PROGRAM(KK, true, true, false); break;           \
    }
#define RBQ_LAUNCH_GROUP_K(KK)                                           \
    if (h->kind & PK_WAITS)                                              \
        RBQ_LAUNCH_PROGRAM(KK, true, true, true);                        \
    else                                                                 \
        RBQ_LAUNCH_PROGRAM(KK, false, true, true)
    const int lmt = (h->kind & PK_MT_MASK) >> PK_MT_SHIFT;
    if (lmt == 1) {
        hipLaunchKernelGGL((gemv_program_kernel<2, RBQ_PROGRAM_RING, false, true, false, 2>), dim3(h->grid),
                           dim3(PG_THREADS), h->lds_bytes, st, hd, h->n_ops, h->checksum, counters, status);
    } else if (lmt == 2) {
        hipLaunchKernelGGL((gemv_program_kernel<2, RBQ_PROGRAM_RING, false, true, false, 4>), dim3(h->grid),
                           dim3(PG_THREADS), h->lds_bytes, st, hd, h->n_ops, h->checksum, counters, status);
    } else if (h->kind & PK_GROUP) {
        if (h->K == 2) {
            RBQ_LAUNCH_GROUP_K(2);
        } else {
            RBQ_LAUNCH_GROUP_K(4);
        }
    } else if (h->K == 1) {
        RBQ_LAUNCH_PROGRAM_K(1);
    } else {
        RBQ_LAUNCH_PROGRAM_K(2);
    }
#undef RBQ_LAUNCH_GROUP_K
#undef RBQ_LAUNCH_PROGRAM_K
#undef RBQ_LAUNCH_PROGRAM
    return hipGetLastError();
}

}  // namespace rbq
