// Device-side helpers for gfx950 (CDNA4): MFMA wrappers, transposed LDS
// reads, cross-half-wave exchange and bf16 packing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D[32x32] += A[32x16] * B[16x32], bf16 in, fp32 accumulate.
// Lane l holds A row l%32, k = 8*(l/32)..+7; B column l%32, same k;
// accumulator register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposed LDS read of 4 bf16. Inside each group of 16 lanes, let lane
// 4e+c load the 4 consecutive values at its address; lane i of the group then
// receives element (i % 4) of the loads of lanes i/4, 4+i/4, 8+i/4, 12+i/4,
// i.e. lane i gets column i of the 4x16 matrix whose row e is the 16 values
// loaded by lanes 4e..4e+3.
__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t* p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}
// The same read at LDS byte address a + imm (imm a compile-time constant, so
// that it becomes the instruction's offset field).
__device__ __forceinline__ bf16x4 lds_read_tr_at(uint32_t a, int imm) {
    typedef __attribute__((address_space(3))) char lds_char;
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_char*)(uintptr_t)a + imm));
    return __builtin_bit_cast(bf16x4, v);
}
// Byte-transposed LDS read (ds_read_b64_tr_b8) at LDS byte address a + imm:
// lanes 2e, 2e+1 of each 16-lane group address row e of an 8-row block, 8
// bytes each, and lane i receives byte i of the 8 rows (row e in byte e).
typedef int i32x2 __attribute__((vector_size(8)));
__device__ __forceinline__ i32x2 lds_read_tr8_at(uint32_t a, int imm) {
    typedef __attribute__((address_space(3))) char lds_char;
    typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)((lds_char*)(uintptr_t)a + imm));
}

__device__ __forceinline__ bf16x8 concat(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Value of x in lane l^32 combined with x: both halves end up with the pair.
// MXFP8 product: acc += (A * 2^(sa-127)) (B * 2^(sb-127)) with E4M3 operands
// of 64 along the contraction. Lane l (row or column l%32, half h = l/32)
// holds 32 bytes: bytes 0-15 are 16 contraction slots of scale block 0,
// bytes 16-31 16 slots of block 1 (which slot is which element is free as
// long as A and B agree), and its scale byte is that of block h of its row.
__device__ __forceinline__ f32x16 mfma_mx(const i32x8& a, const i32x8& b, int sa, int sb, const f32x16& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Four fp32 values / scale as E4M3 codes packed in one dword (value i in
// byte i; round to nearest even; callers keep |value / scale| <= 448).
__device__ __forceinline__ uint32_t pack4_fp8(float x0, float x1, float x2, float x3, float scale) {
    s16x2 w = {0, 0};
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, x0, x1, scale, false);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, x2, x3, scale, true);
    return __builtin_bit_cast(uint32_t, w);
}

__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 to_bf16x8(f32x8 x) { return __builtin_convertvector(x, bf16x8); }
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *(const u32x4*)p);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima): wait for all
// vector memory operations of this wave. Placed before a loop whose body
// issues prefetch loads, it keeps the compiler from conservatively waiting on
// those prefetches inside the loop (its per-register wait tracking is merged
// over the back edge).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): all but this wave's N most recent vector memory
// operations have completed (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_keep() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Executed-tile log of debug builds (compiled with JFA_TILE_LOG; nothing
// otherwise). Thread 0 of worker w's workgroup writes the n-th tile the
// worker takes as record n of its area, log + w * (8 + 8 cap): area[0] is
// the number of tiles taken so far (n + 1), record n is the 8 int32 at
// area + 8 + 8 n (records past cap are counted, not stored). The wave then
// waits for the stores, so the kernel's counted waits on its own copies
// still see only those copies.
struct TileLogRec {
    int pass, worker, b, h, t, work, blocks, flags;
};
__device__ __forceinline__ void tile_log(int32_t* log, int cap, int n, const TileLogRec& r) {
#ifdef JFA_TILE_LOG
    if (log != nullptr) {
        if (threadIdx.x == 0) {
            int32_t* area = log + (int64_t)r.worker * (8 + 8 * (int64_t)cap);
            if (n < cap) {
                int4* rec = (int4*)(area + 8 + 8 * (int64_t)n);
                rec[0] = make_int4(r.pass, r.worker, r.b, r.h);
                rec[1] = make_int4(r.t, r.work, r.blocks, r.flags);
            }
            area[0] = n + 1;
        }
        wait_vmem();
    }
#else
    (void)log, (void)cap, (void)n, (void)r;
#endif
}
#ifdef JFA_TILE_LOG
constexpr bool kTileLog = true;
#else
constexpr bool kTileLog = false;
#endif
// flag bits of a record: the plan's indices checked against the problem
constexpr int kLogBadBatch = 1, kLogBadHead = 2, kLogBadTile = 4, kLogBadStream = 8;

// Scheduling hint for a run of N MFMAs each fed by R LDS operand reads:
// issue the reads of the first A MFMAs, then alternate one MFMA with the
// reads of one more, then the last A MFMAs. Without it the scheduler keeps a
// single read in flight and every MFMA waits out a full LDS latency. Only
// orders the reads and MFMAs of the current scheduling region; other
// instructions move freely.
template <int N, int A, int R = 1>
__device__ __forceinline__ void pipeline_reads_mfma() {
    constexpr int kMfma = 0x008, kDsRead = 0x100;
    __builtin_amdgcn_sched_group_barrier(kDsRead, A * R, 0);
#pragma unroll
    for (int j = 0; j < N - A; ++j) {
        __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kDsRead, R, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kMfma, A, 0);
}

// Orders a wave's LDS writes before its following LDS reads of what other
// lanes of the same wave wrote (and the reads before later overwrites).
// Without it such cross-lane traffic is a data race to the compiler, which
// may then move the reads, e.g. into a branch only some lanes take.
__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The value of x, opaque to the optimiser: values derived from it are
// recomputed where they are used instead of being hoisted out of loops (and
// then spilled when registers are short).
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Load of a wave-uniform value from memory the kernel never writes (plans,
// offsets), through the constant address space so that it becomes a scalar
// load: a vector load would need a vmcnt wait, which also waits for every
// copy in flight.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p) {
    return *(const __attribute__((address_space(4))) T*)p;
}

// Atomic increment of *p by lane 0 alone (the exec mask is narrowed inside
// the asm, so the surrounding code stays free of lane-divergent branches),
// returning the old value in lane 0. The asm waits for the value (vmcnt(0):
// this also waits for the wave's earlier vector memory operations). It has
// to: the compiler takes an asm output as ready when the asm ends, and may
// copy or spill the register right there, before any later wait, which
// would read it before the atomic has written it. (A compiler-visible
// atomic is tracked correctly but, restricted to one lane, turns the
// loader's wave-uniform state into per-lane state in the generated code.)
__device__ __forceinline__ int atomic_inc_lane0(int* p) {
    int r;
    uint64_t saved;
    asm volatile(
        "s_mov_b64 %1, exec\n\t"
        "s_mov_b64 exec, 1\n\t"
        "global_atomic_add %0, %2, %3, off sc0\n\t"
        "s_waitcnt vmcnt(0)\n\t"
        "s_mov_b64 exec, %1"
        : "=&v"(r), "=&s"(saved)
        : "v"(p), "v"(1)
        : "memory");
    return r;
}

// Persistent worker of this workgroup. Workgroup ids are dealt round-robin to
// the 8 XCDs; mapping consecutive workers to the same XCD puts tiles dealt
// next to each other (e.g. the Q tiles of one sequence and head, which read
// the same K/V) behind the same L2.
__device__ __forceinline__ int worker_id(int num_workers) {
    const int bid = blockIdx.x;
    if ((num_workers & 7) == 0) return (bid & 7) * (num_workers >> 3) + (bid >> 3);
    return bid;
}

}  // namespace jfa
