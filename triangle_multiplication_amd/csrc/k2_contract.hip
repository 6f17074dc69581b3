// k2_contract.hip -- the triangle contraction: for every (batch, channel) slab,
// o[i][j] = sum_k a_cm[i][k] * b_cm[j][k] over k in [0, N), fp32 accumulation
// on matrix cores, one rounding to the storage type at the end.
//
// The projection kernel stores a and b channel-major with k contiguous for both
// directions (the incoming direction's transpose is folded into that store), so
// this is always an "NT" product of two K-contiguous operands.  fp32 operand
// slabs are plain [row][k]; bf16 slabs are K-blocked (kblk_off: blocks of 32 k
// holding all rows), so every K-step reads whole contiguous runs.  o is always
// plain [i][j].  bf16 runs the persistent kernel k2_contract_ppp at every N;
// fp32 the register-staged kernel k2_contract.
//
// k2_contract (fp32): a 256-thread workgroup (4 waves in a 2 x 2 grid) owns a BM x BN tile
// of o; each wave owns (BM/2) x (BN/2) as 16 x 16 MFMA blocks.  K advances 128
// bytes per stage (64 bf16 / 32 fp32), staged through double-buffered LDS with
// the chunk swizzle of trimul_device.hpp; global loads for stage k+1 are in
// flight while stage k is multiplied.  Rows or K chunks past N read as zero, and
// stores past N are skipped, so any N that is a multiple of 8 works.
#include "trimul_device.hpp"
#include "trimul_launch.hpp"

namespace trimul {

template <typename T, int BM, int BN>
__global__ __launch_bounds__(256) void k2_contract(const T* __restrict__ A, const T* __restrict__ Bm,
                                                   T* __restrict__ O, size_t o_stride, int bc0, int N,
                                                   int tiles_j)
{
    constexpr int CE = Elem<T>::CE;
    constexpr int KCH = 8;                  // 16-byte chunks per tile row per stage
    constexpr int BK = KCH * CE;            // K elements per stage
    constexpr int WM = BM / 2, WN = BN / 2; // wave tile
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int A_LD = BM * KCH / 256;    // chunks each thread loads per stage
    constexpr int B_LD = BN * KCH / 256;
    __shared__ u32x4 lds[2][(BM + BN) * KCH];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const size_t slab = (size_t)N * N;
    // Tile order.  Workgroups are handed to the 8 XCDs round-robin by id, so id g
    // runs on XCD g % 8.  Give each XCD a contiguous range of logical tiles
    // (channel-major), and inside a channel walk groups of GM tile rows column by
    // column: the ~32 tiles an XCD runs at once then share GM row panels of a and
    // a few column panels of b in that XCD's L2.
    const int tiles_i = (N + BM - 1) / BM;
    const int per_bc = tiles_i * tiles_j;
    const unsigned total = gridDim.x;                 // B*C*per_bc, a multiple of 8
    const unsigned g = blockIdx.x;
    const unsigned logical = (g & 7u) * (total >> 3) + (g >> 3);
    const size_t bc = logical / per_bc;
    const int t = (int)(logical % per_bc);
    constexpr int GM = 4;
    const int group = t / (GM * tiles_j);
    const int first_i = group * GM;
    const int gm = min(GM, tiles_i - first_i);
    const int ti = first_i + (t % (GM * tiles_j)) % gm;
    const int tj = (t % (GM * tiles_j)) / gm;
    static_assert(sizeof(T) == 4, "bf16 operands are K-blocked and use k2_contract_ppp");
    const T* Ab = A + (bc0 + bc) * slab;
    const T* Bb = Bm + (bc0 + bc) * slab;
    T* Ob = O + bc * o_stride;
    auto opoff = [&](int row, int k) -> size_t { return (size_t)row * N + k; };
    const int i0 = ti * BM, j0 = tj * BN;

    u32x4 ra[A_LD], rb[B_LD];
    const u32x4 zero = {0u, 0u, 0u, 0u};

    auto gload = [&](int k0) {
#pragma unroll
        for (int it = 0; it < A_LD; ++it) {
            int q = tid + 256 * it, row = q >> 3, c = q & 7;
            int gi = i0 + row, gk = k0 + c * CE;
            ra[it] = (gi < N && gk < N) ? ld16(Ab + opoff(gi, gk)) : zero;
        }
#pragma unroll
        for (int it = 0; it < B_LD; ++it) {
            int q = tid + 256 * it, row = q >> 3, c = q & 7;
            int gj = j0 + row, gk = k0 + c * CE;
            rb[it] = (gj < N && gk < N) ? ld16(Bb + opoff(gj, gk)) : zero;
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int it = 0; it < A_LD; ++it) {
            int q = tid + 256 * it, row = q >> 3, c = q & 7;
            lds[buf][row * KCH + swz(row, c)] = ra[it];
        }
#pragma unroll
        for (int it = 0; it < B_LD; ++it) {
            int q = tid + 256 * it, row = q >> 3, c = q & 7;
            lds[buf][BM * KCH + row * KCH + swz(row, c)] = rb[it];
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int m = 0; m < FM; ++m)
#pragma unroll
        for (int n = 0; n < FN; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (N + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
        for (int kg = 0; kg < KCH / 4; ++kg) {
            const int c = kg * 4 + (lane >> 4);
            u32x4 fa[FM], fb[FN];
#pragma unroll
            for (int m = 0; m < FM; ++m) {
                int row = wm * WM + m * 16 + (lane & 15);
                fa[m] = lds[buf][row * KCH + swz(row, c)];
            }
#pragma unroll
            for (int n = 0; n < FN; ++n) {
                int row = wn * WN + n * 16 + (lane & 15);
                fb[n] = lds[buf][BM * KCH + row * KCH + swz(row, c)];
            }
            // Operands swapped (b rows as the MFMA's A): each lane's four results
            // are four consecutive j of one i, so the store is one 4-element run.
#pragma unroll
            for (int m = 0; m < FM; ++m)
#pragma unroll
                for (int n = 0; n < FN; ++n) acc[m][n] = Elem<T>::mma(fb[n], fa[m], acc[m][n]);
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int m = 0; m < FM; ++m) {
        const int i = i0 + wm * WM + m * 16 + (lane & 15);
#pragma unroll
        for (int n = 0; n < FN; ++n) {
            const int j = j0 + wn * WN + n * 16 + 4 * (lane >> 4);
            if (i < N && j < N) Elem<T>::store4(Ob, (size_t)i * N + j, acc[m][n]);
        }
    }
}

// ---------------------------------------------------------------------------
// Large-N bf16 path: 256 x 256 tiles fed by LDS DMA.
//
// K advances 32 per step.  The operand rows of a step (64 bytes each, 256 rows
// of a and 256 of b = 32 KB) live in a ring of LDS slots filled by
// buffer_load ... lds (global -> LDS without registers).  K chunks past N and
// steps past the workgroup's last tile are pushed out of the buffer's range
// and read as zero, so the ring runs past the last step without tail code;
// tile rows past N read zeros or other rows' data, which reach only outputs
// that are not stored.
//
// LDS layout of one operand in one slot (256 rows x 4 chunks of 16 bytes):
// rows are paired into 128-byte lines, line L = row / 2 holds the 16-byte slot
// ((row % 2) * 4 + chunk) ^ (L % 8).  For the MFMA fragment read (lane l: row
// l % 16 of a 16-row block, chunk l / 16) this is free of LDS bank conflicts on
// gfx950 (measured: 4 cycles per ds_read_b128, the rate of a contiguous read),
// and each 1 KB DMA write is contiguous.
// The compiler does not order LDS DMA against ds_read, so every hand-off is an
// explicit s_waitcnt + s_barrier.
// ---------------------------------------------------------------------------
namespace k2big {
constexpr int BM = 256, BN = 256, BK = 32;
constexpr int ROWB = 64;                       // bytes of one operand row per step
constexpr int OPB = BM * ROWB;                 // bytes of one operand per slot (16 KB)
constexpr int STB = 2 * OPB;                   // bytes per slot (a and b)

__device__ inline int slot_off(int row, int chunk)
{
    const int L = row >> 1;
    return L * 128 + (((((row & 1) << 2) | chunk) ^ (L & 7)) << 4);
}
}  // namespace k2big

#define TRIMUL_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Persistent kernel: one 512-thread workgroup per CU walks its tiles g, g + G,
// ... in an XCD-aware order (workgroup g runs on XCD g % 8).  Two orders:
//  order 0: the launch's tiles are cut into 8 contiguous bands, one per XCD;
//  order 1: each round of G consecutive tiles (one per workgroup) is cut into
//           8 contiguous blocks, one per XCD, so all XCDs work on the same few
//           channels at once and what one XCD's L2 misses, the last-level
//           cache (shared by all XCDs) still holds from the others.
// Within a channel, tiles are walked in groups of gm row panels, column by
// column, so the ~32 tiles an XCD runs at once share K-slices of a few panels
// in its L2 (gm = 8 measured best against 1, 2, 4 and 16 at N = 4096 with
// order 0).
//
// k2_contract_ppp below runs one K-step per phase (the 128-row-tile plans);
// k2_contract_pp2 after it runs two (256-row tiles) on the same scheme.
// 8 waves in a 2 x 4 grid, each owning a 128 x 64 block of the tile (8 x 4
// MFMA tiles, 128 accumulators per lane); the two waves that share a SIMD
// (wave w and w + 4) run half a step apart ("ping-pong").  Each wave
// alternates a memory phase M_k (read step k's fragments from LDS, issue its
// share of step k+3's DMA) and a compute phase C_k (32 MFMAs); group 0 (waves
// 0-3) is one phase ahead of group 1 (waves 4-7), so in every phase one wave of
// each SIMD multiplies while the other loads, and phases are separated by one
// workgroup barrier.  Steps are numbered across the workgroup's tiles.
//
// Phase p: group 0 runs M_{p/2} (p even) or C_{(p-1)/2} (p odd); group 1 runs
// the same one phase later.  Invariants (NSP = 4 slots, DMA three steps ahead):
//  - step k's slot is read in phases 2k (group 0) and 2k+1 (group 1); every
//    wave's DMA share of step k was issued at least four phases earlier, and
//    before each barrier a wave waits until at most two of its steps are in
//    flight, so step k has landed for everyone when phase 2k starts;
//  - step k+3's DMA overwrites step k-1's slot, first in phase 2k, after the
//    barrier that ends phase 2k-1 where the last reader (group 1) finished; a
//    memory phase ends with lgkmcnt(0) so its reads are complete at that barrier.
// Group 1 takes one extra barrier at the start and group 0 one at the end, so
// every wave executes the same number of barriers.
//
// The DMA ring is never drained between tiles: the next tile's first steps
// are in flight while the current one finishes, and a tile's stores overlap
// the next tile's multiplies.  A wave stores its block and clears its
// accumulators right after the compute phase of a tile's last step; both
// groups do this at the same point of their own phase sequence, so every wave
// still executes the same barriers.
//
// Masked calls pass a table of live K-step ranges per row tile: a tile runs
// only the K-steps where both its A rows and its B rows can be nonzero (every
// skipped product is an exact zero, so the sums are unchanged); a tile with
// no such step runs one step of zeros (the DMA is pushed out of range) and
// stores its zeros.  Step counts per tile are the same for every wave of the
// workgroup, so the barrier sequence stays uniform.  The table also lists each
// batch's tile pairs live-first, and the launch's tiles are numbered so that
// every channel's live pairs come before any dead pair: rounds of live tiles
// then stay uniform and the workgroups of an XCD stay in step (a dead tile
// among live ones lets its workgroup run ahead and stop sharing panels).
//
// Operands are K-blocked (kblk_off): a step's 256 rows of one operand are one
// contiguous 16 KB run, and each DMA instruction reads one contiguous
// kilobyte (16 rows x 64 bytes).  With row-major operands the same step reads
// 256 half cache lines 2N bytes apart, which measured 12 % slower overall.
struct K2PArgs {
    const bf16* A;        // operand slabs [B*C][aslab], K-blocked
    const bf16* Bm;
    bf16* O;              // output of local slab t at O + t * o_stride
    size_t o_stride;
    const int* ranges;    // mask table: [B][tiles][2] live K-step ranges, or null
    const int* hdr;       //   its header ([0] = live pairs of the fullest batch)
    const unsigned* pairs;//   its pair lists [B][tiles^2]
    int N, C, total;      // total = tiles of this launch (a multiple of 8)
    int bc0;              // first operand slab of this launch
    int order, gm;        // Plan
};

// MK: the launch carries a mask table (args.ranges and the pair lists); the
// unmasked instantiation runs every tile over all its K-steps with no table
// reads and no per-tile range bookkeeping.
template <int NSP, int TB, bool MK>
__global__ __launch_bounds__(512) void k2_contract_ppp(K2PArgs args)
{
    using namespace k2big;
    static_assert(TB == 256 || TB == 128, "tile sides");
    constexpr int NW = 8;
    constexpr int DPO = OPB / 1024 / NW;            // DMA instructions per wave per operand (2)
    constexpr int DPS = 2 * DPO;                    // per wave per step
    constexpr int DIST = NSP - 1;                   // DMA runs this many steps ahead
    constexpr int KH = BM / TB;                     // 32-key blocks per step (1 or 2)
    constexpr int RG = TB / 16;                     // 16-row groups of one key block
    constexpr int WM = TB / 2, WN = TB / 4;         // a wave's block of the tile
    constexpr int MB = WM / 16, NB = WN / 16;       // its 16 x 16 MFMA blocks
    static_assert(NB % 2 == 0 && RG % 2 == 0, "paired column blocks and row groups");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NSP * STB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;        // group = wm
    const int N = args.N, total = args.total;
    const int tiles = (N + TB - 1) / TB;
    const int per_bc = tiles * tiles;
    const int G = gridDim.x, g = blockIdx.x;
    const int n_my = (total - g + G - 1) / G;       // tiles of this workgroup (g < total)
    const int nk = (N + BK * KH - 1) / (BK * KH);   // steps of a whole tile
    // Live-first pair lists exist for 256-row tiles only; 128-row tiles walk
    // the plain order and take the key range of the 256-row tiles holding them.
    constexpr bool use_pairs = TB == 256 && MK;

    // Tile tl of this workgroup: virtual block vb = g + tl*G through the
    // order's map, a bijection of [0, total) (total and G are multiples of 8),
    // which keeps every tile of workgroup g on g's XCD.
    auto logical_of = [&](unsigned vb) -> unsigned {
        if (args.order == 0) return (vb & 7u) * ((unsigned)total >> 3) + (vb >> 3);
        const unsigned r = vb / (unsigned)G, gg = vb - r * (unsigned)G;
        const unsigned rem = (unsigned)total - r * (unsigned)G;
        const unsigned R = rem < (unsigned)G ? rem : (unsigned)G;   // tiles of round r
        return r * (unsigned)G + (gg & 7u) * (R >> 3) + (gg >> 3);
    };
    // Masked: the first nbc * nl logical tiles are slots [0, nl) of every
    // slab's pair list, the rest slots [nl, tiles^2).
    const unsigned nl = use_pairs ? (unsigned)args.hdr[0] : 0u;
    const unsigned nbc_l = (unsigned)total / (unsigned)per_bc;
    auto tile_geo = [&](int tl, size_t& bc, int& ti, int& tj) {
        const unsigned logical = logical_of((unsigned)g + (unsigned)tl * (unsigned)G);
        if (use_pairs) {
            unsigned p;
            if (logical < nbc_l * nl) {
                bc = logical / nl;
                p = logical % nl;
            } else {
                const unsigned r = logical - nbc_l * nl, nd = (unsigned)per_bc - nl;
                bc = r / nd;
                p = nl + r % nd;
            }
            const unsigned e = args.pairs[((size_t)args.bc0 + bc) / (size_t)args.C * per_bc + p];
            ti = (int)(e & 0xffffu);
            tj = (int)(e >> 16);
            return;
        }
        bc = logical / per_bc;
        const int t = (int)(logical % per_bc);
        const int GM = args.gm;
        const int first_i = (t / (GM * tiles)) * GM;
        const int gm = min(GM, tiles - first_i);
        ti = first_i + (t % (GM * tiles)) % gm;
        tj = (t % (GM * tiles)) / gm;
    };
    // K-steps of tile (bc, ti, tj): [klo, klo + kn); kn >= 1, and dead tiles
    // (no live step) run one step that reads zeros.  The table's ranges are in
    // 32-key blocks of 256-row tiles; a step of KH blocks is run if any of its
    // blocks is live.
    const int t256 = (N + BM - 1) / BM;
    // The values are uniform over the workgroup; readfirstlane keeps them in
    // scalar registers, so the per-step cursor and loop tests stay scalar.
    auto krange = [&](size_t bc, int ti, int tj, int& klo, int& kn, bool& live) {
        if constexpr (!MK) {
            klo = 0;
            kn = nk;
            live = true;
        } else {
            const int b = (int)(((size_t)args.bc0 + bc) / (size_t)args.C);
            const int* r = args.ranges + (size_t)b * t256 * 2;
            const int ui = ti * TB / BM, uj = tj * TB / BM;
            const int lo = __builtin_amdgcn_readfirstlane(max(r[2 * ui], r[2 * uj]));
            const int hi = __builtin_amdgcn_readfirstlane(min(r[2 * ui + 1], r[2 * uj + 1]));
            live = lo < hi;
            klo = live ? lo / KH : 0;
            kn = live ? (hi + KH - 1) / KH - lo / KH : 1;
        }
    };

    // Operand slab: [nk][N][32] bf16.  A slot holds, per operand, KH key
    // blocks of TB rows (16 KB either way).  DMA instruction q of a wave fills
    // kilobyte 2 wave + q of the operand's part: key block kh_w = (2 wave) / RG
    // of the step, rows 16 ((2 wave + q) % RG) .. +15 of the tile, one
    // contiguous kilobyte of the slab; lane l reads row dr, chunk dc (the slot
    // swizzle is applied by choosing which lane reads which chunk).
    const size_t aslab = ab_slab_elems(DType::BF16, N);
    const unsigned nrec = (unsigned)(aslab * sizeof(bf16));
    const int dpos = (lane & 7) ^ (lane >> 3);
    const int dr = 2 * (lane >> 3) + (dpos >> 2), dc = dpos & 3;
    constexpr unsigned qstride = 16u * ROWB;
    const unsigned kstride = (unsigned)N * ROWB;    // bytes per K-block
    const int kh_w = KH == 1 ? 0 : __builtin_amdgcn_readfirstlane((2 * wave) / RG);   // its key block of a step
    const int g32 = ((2 * wave) % RG) / 2;          // its 32-row group of the tile
    const unsigned lane_off = (unsigned)(32 * g32 + dr) * ROWB + dc * 16u;
    // B rows are loaded permuted within each 32-row group: slot row 16 h + r
    // (h = 0, 1; r = 0..15) holds tile row 8 (r / 4) + 4 h + r % 4.  After the
    // MFMAs of blocks 2p and 2p + 1, lane group g then holds the results for
    // rows 32 p + 8 g .. + 7 of its wave's columns, eight consecutive j of one
    // i, stored as one 16-byte run.  Instruction q of a wave fills slot rows
    // 16 (2 g32 + q) .. + 15, i.e. h = q and group g32.
    static_assert(DPO == 2, "B row permutation assumes two DMA instructions per operand per wave");
    const unsigned lane_off_b = (unsigned)(32 * g32 + 8 * (dr >> 2) + (dr & 3)) * ROWB + dc * 16u;

    // DMA cursor: the next step to load is step ikk of tile itl (K-step
    // iklo + ikk; its first key ik0 and byte offset ikb advance by one step
    // per issue).  The tile's buffer descriptors, row offsets and K range are
    // recomputed only when the cursor enters a new tile; past the workgroup's
    // last tile, in dead tiles and for K-chunks past N the offset is pushed
    // beyond the buffer's range, so the DMA reads zeros.
    int itl = 0, ikk = 0, iklo = 0, ikn = 1, ik0 = 0;
    unsigned ikb = 0;
    __amdgpu_buffer_rsrc_t ra, rb;
    unsigned oa_t = 0, ob_t = 0;
    bool ilive = true;
    auto set_tile = [&]() {
        const bool have = itl < n_my;
        size_t bc; int ti, tj;
        tile_geo(have ? itl : 0, bc, ti, tj);
        bool klive;
        krange(bc, ti, tj, iklo, ikn, klive);
        ilive = have && klive;
        const size_t sb = (size_t)args.bc0 + bc;
        ra = __builtin_amdgcn_make_buffer_rsrc((void*)(args.A + sb * aslab), 0, nrec, 0x00020000);
        rb = __builtin_amdgcn_make_buffer_rsrc((void*)(args.Bm + sb * aslab), 0, nrec, 0x00020000);
        oa_t = lane_off + (unsigned)(ti * TB) * ROWB;
        ob_t = lane_off_b + (unsigned)(tj * TB) * ROWB;
        const int kk = iklo * KH + kh_w;                // key block of the tile's first step
        ik0 = kk * BK;
        ikb = (unsigned)kk * kstride;
    };
    set_tile();
    int isl = 0;                                    // ring slot of the next step
    auto issue = [&]() {
        unsigned char* st = smem + isl * STB + wave * DPO * 1024;
        const unsigned kb = ikb;
        const unsigned kpen = (ilive && ik0 + dc * 8 < N) ? 0u : 0x80000000u;
        ik0 += KH * BK;
        ikb += (unsigned)KH * kstride;
#pragma unroll
        for (int q = 0; q < DPO; ++q) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, TRIMUL_LDS_PTR(st + q * 1024), 16,
                                                     (oa_t + q * qstride + kb) | kpen, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, TRIMUL_LDS_PTR(st + OPB + q * 1024), 16,
                                                     (ob_t + q * 4u * ROWB + kb) | kpen, 0, 0, 0);
        }
        if (++isl == NSP) isl = 0;
        if (++ikk == ikn) { ikk = 0; ++itl; set_tile(); }
    };

    // Fragments: key block kh of a slot starts TB rows (TB * 64 bytes) after
    // block kh - 1 in each operand's part.
    const int rchunk = lane >> 4;
    const int fa_base = slot_off(wm * WM + (lane & 15), rchunk);
    const int fb_base = OPB + slot_off(wn * WN + (lane & 15), rchunk);

    f32x4 acc[MB][NB];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 fa[KH][MB], fb[KH][NB];
    auto barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

#pragma unroll
    for (int s0 = 0; s0 < DIST; ++s0) issue();
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((DIST - 1) * DPS));   // own share of step 0 landed
    barrier();                                          // ... everyone's
    if (wm == 1) barrier();                             // group 1 starts one phase late

    int kin = 0;                                        // step within the current tile
    int tl = 0;
    int nk_cur;                                         // steps of tile tl
    {
        size_t bc; int ti, tj, klo; bool lv;
        tile_geo(0, bc, ti, tj);
        krange(bc, ti, tj, klo, nk_cur, lv);
    }
    int rsl = 0;                                        // ring slot of the current step
    for (;;) {
        // M_s
        const unsigned char* st = smem + rsl * STB;
        if (++rsl == NSP) rsl = 0;
#pragma unroll
        for (int kh = 0; kh < KH; ++kh) {
#pragma unroll
            for (int m = 0; m < MB; ++m)
                fa[kh][m] = *reinterpret_cast<const u32x4*>(st + kh * TB * ROWB + fa_base + m * 1024);
#pragma unroll
            for (int n = 0; n < NB; ++n)
                fb[kh][n] = *reinterpret_cast<const u32x4*>(st + kh * TB * ROWB + fb_base + n * 1024);
        }
        issue();                                        // step s + DIST
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds0((DIST - 1) * DPS));
        barrier();
        // C_s.  Operands swapped (b rows as the MFMA's A): each lane's four
        // results are four consecutive j of one i.
#pragma unroll
        for (int kh = 0; kh < KH; ++kh)
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int n = 0; n < NB; ++n) acc[m][n] = Elem<bf16>::mma(fb[kh][n], fa[kh][m], acc[m][n]);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm((DIST - 1) * DPS));
        barrier();
        if (++kin == nk_cur) {
            // Tile tl complete: store this wave's block and start the next.
            size_t bc; int ti, tj;
            tile_geo(tl, bc, ti, tj);
            const int i0 = ti * TB, j0 = tj * TB;
            bf16* Ob = args.O + bc * args.o_stride;
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                const int i = i0 + wm * WM + m * 16 + (lane & 15);
#pragma unroll
                for (int p = 0; p < NB / 2; ++p) {
                    // j .. j + 7 (8 divides N, so all or none exist)
                    const int j = j0 + wn * WN + 32 * p + 8 * (lane >> 4);
                    bf16x8 h;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        h[e] = (bf16)acc[m][2 * p][e];
                        h[4 + e] = (bf16)acc[m][2 * p + 1][e];
                    }
                    if (i < N && j < N) *reinterpret_cast<bf16x8*>(Ob + (size_t)i * N + j) = h;
                    acc[m][2 * p] = f32x4{0.f, 0.f, 0.f, 0.f};
                    acc[m][2 * p + 1] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
            kin = 0;
            if (++tl == n_my) break;
            size_t nbc; int nti, ntj, klo; bool lv;
            tile_geo(tl, nbc, nti, ntj);
            krange(nbc, nti, ntj, klo, nk_cur, lv);
        }
    }
    if (wm == 0) barrier();                             // balance group 1's extra barrier
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));          // no DMA may outlive the workgroup
}

// ---------------------------------------------------------------------------
// Two K-steps per phase (256-row tiles).  The same tiles, walk, key ranges,
// fragment layout and MFMA order per output as the one-step kernel above
// would use at 256-row tiles (so the same bits as every other plan: each
// output sums its keys in the same MFMA sequence), but each memory phase reads the fragments of two steps
// and each compute phase runs 64 MFMAs, so the per-phase cost of the barrier,
// the waits and the LDS latency is paid once per two steps.  A copy of the
// one-step kernel that ran every MFMA twice per phase reached the rate of an
// MFMA-only loop, which is what this form aims at.
//
// Ring: 5 slots of one step (160 KB), step k in slot k % 5.  Super-step u is
// steps 2u and 2u + 1; phase p: group 0 runs M_{p/2} (p even) or C_{(p-1)/2};
// group 1 the same one phase later.  Each group loads whole steps: group 0 the
// odd steps (step 2u + 3 in M_u), group 1 the even ones (step 2u + 4 in M_u),
// each wave eight 1 KB DMA instructions (rows 64 w' .. + 63 of both operands,
// w' = wave % 4).  Invariants:
//  - step 2u + 3 overwrites step 2u - 2 and step 2u + 4 step 2u - 1 (super-step
//    u - 1), first in phase 2u, after the barrier ending phase 2u - 1 where
//    group 1 finished reading them (memory phases end with lgkmcnt(0));
//  - super-step v is read from phase 2v on; its odd step was loaded by group 0
//    in phase 2v - 2 and its even step by group 1 in phase 2v - 3.  Group 0
//    waits for all its loads at the end of each compute phase (phase 2v - 1),
//    group 1 for all but its newest step at the end of each phase, so both
//    steps have landed for everyone when phase 2v starts.
// A tile's step count is rounded up to even; the extra step reads zeros (its
// DMA is pushed out of the buffer's range), which adds exact zeros.
// ---------------------------------------------------------------------------
template <bool MK>
__global__ __launch_bounds__(512) void k2_contract_pp2(K2PArgs args)
{
    using namespace k2big;
    constexpr int NSP = 5, TB = 256;
    constexpr int NW = 8;
    constexpr int RG = TB / 16;                     // 16-row groups of the tile
    constexpr int WM = TB / 2, WN = TB / 4;         // a wave's block of the tile
    constexpr int MB = WM / 16, NB = WN / 16;       // its 16 x 16 MFMA blocks
    constexpr int DPW = 8;                          // DMA instructions per loading wave per step
    static_assert(NB % 2 == 0 && RG % 2 == 0 && OPB == 16 * 1024, "paired column blocks, 16 KB operands");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NSP * STB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;        // group = wm
    const int N = args.N, total = args.total;
    const int tiles = (N + TB - 1) / TB;
    const int per_bc = tiles * tiles;
    const int G = gridDim.x, g = blockIdx.x;
    const int n_my = (total - g + G - 1) / G;       // tiles of this workgroup (g < total)
    const int nk = (N + BK - 1) / BK;               // steps of a whole tile
    constexpr bool use_pairs = MK;

    auto logical_of = [&](unsigned vb) -> unsigned {
        if (args.order == 0) return (vb & 7u) * ((unsigned)total >> 3) + (vb >> 3);
        const unsigned r = vb / (unsigned)G, gg = vb - r * (unsigned)G;
        const unsigned rem = (unsigned)total - r * (unsigned)G;
        const unsigned R = rem < (unsigned)G ? rem : (unsigned)G;
        return r * (unsigned)G + (gg & 7u) * (R >> 3) + (gg >> 3);
    };
    const unsigned nl = use_pairs ? (unsigned)args.hdr[0] : 0u;
    const unsigned nbc_l = (unsigned)total / (unsigned)per_bc;
    auto tile_geo = [&](int tl, size_t& bc, int& ti, int& tj) {
        const unsigned logical = logical_of((unsigned)g + (unsigned)tl * (unsigned)G);
        if (use_pairs) {
            unsigned p;
            if (logical < nbc_l * nl) {
                bc = logical / nl;
                p = logical % nl;
            } else {
                const unsigned r = logical - nbc_l * nl, nd = (unsigned)per_bc - nl;
                bc = r / nd;
                p = nl + r % nd;
            }
            const unsigned e = args.pairs[((size_t)args.bc0 + bc) / (size_t)args.C * per_bc + p];
            ti = (int)(e & 0xffffu);
            tj = (int)(e >> 16);
            return;
        }
        bc = logical / per_bc;
        const int t = (int)(logical % per_bc);
        const int GM = args.gm;
        const int first_i = (t / (GM * tiles)) * GM;
        const int gm = min(GM, tiles - first_i);
        ti = first_i + (t % (GM * tiles)) % gm;
        tj = (t % (GM * tiles)) / gm;
    };
    const int t256 = (N + BM - 1) / BM;
    // K-steps of tile (bc, ti, tj): [klo, klo + kn), kn >= 1 (see the one-step kernel).
    auto krange = [&](size_t bc, int ti, int tj, int& klo, int& kn, bool& live) {
        if constexpr (!MK) {
            klo = 0;
            kn = nk;
            live = true;
        } else {
            const int b = (int)(((size_t)args.bc0 + bc) / (size_t)args.C);
            const int* r = args.ranges + (size_t)b * t256 * 2;
            const int lo = __builtin_amdgcn_readfirstlane(max(r[2 * ti], r[2 * tj]));
            const int hi = __builtin_amdgcn_readfirstlane(min(r[2 * ti + 1], r[2 * tj + 1]));
            live = lo < hi;
            klo = live ? lo : 0;
            kn = live ? hi - lo : 1;
        }
    };

    // DMA lanes: lane l reads row dr, chunk dc of a 16-row kilobyte (the slot
    // swizzle is applied by choosing which lane reads which chunk).  Loading
    // wave w' fills kilobytes 4 w' + i (i = 0..3) of both operands: A rows
    // 16 j + dr of kilobyte j; B rows permuted within each 32-row group (slot
    // row 16 h + r holds tile row 8 (r / 4) + 4 h + r % 4) as in the one-step
    // kernel, so a lane stores eight consecutive j of one i.
    const size_t aslab = ab_slab_elems(DType::BF16, N);
    const unsigned nrec = (unsigned)(aslab * sizeof(bf16));
    const int dpos = (lane & 7) ^ (lane >> 3);
    const int dr = 2 * (lane >> 3) + (dpos >> 2), dc = dpos & 3;
    const unsigned kstride = (unsigned)N * ROWB;    // bytes per K-block
    const int wq = wave & 3;                        // w'
    const unsigned lane_off = (unsigned)(64 * wq + dr) * ROWB + dc * 16u;
    const unsigned lane_off_b = (unsigned)(64 * wq + 8 * (dr >> 2) + (dr & 3)) * ROWB + dc * 16u;

    // DMA cursor over the workgroup's step sequence (tiles back to back, each
    // padded to an even step count): step ikk of tile itl, first key ik0,
    // byte offset ikb, ring slot isl.
    int itl = 0, ikk = 0, ikn = 1, ikn2 = 2, ik0 = 0, isl = 0;
    unsigned ikb = 0;
    __amdgpu_buffer_rsrc_t ra, rb;
    unsigned oa_t = 0, ob_t = 0;
    bool ilive = true;
    auto set_tile = [&]() {
        const bool have = itl < n_my;
        size_t bc; int ti, tj, iklo;
        tile_geo(have ? itl : 0, bc, ti, tj);
        bool klive;
        krange(bc, ti, tj, iklo, ikn, klive);
        ikn2 = (ikn + 1) & ~1;
        ilive = have && klive;
        const size_t sb = (size_t)args.bc0 + bc;
        ra = __builtin_amdgcn_make_buffer_rsrc((void*)(args.A + sb * aslab), 0, nrec, 0x00020000);
        rb = __builtin_amdgcn_make_buffer_rsrc((void*)(args.Bm + sb * aslab), 0, nrec, 0x00020000);
        oa_t = lane_off + (unsigned)(ti * TB) * ROWB;
        ob_t = lane_off_b + (unsigned)(tj * TB) * ROWB;
        ik0 = iklo * BK;
        ikb = (unsigned)iklo * kstride;
    };
    set_tile();
    auto advance = [&]() {
        ik0 += BK;
        ikb += kstride;
        if (++isl == NSP) isl = 0;
        if (++ikk == ikn2) { ikk = 0; ++itl; set_tile(); }
    };
    auto issue = [&]() {                            // this wave's share of the cursor's step
        unsigned char* st = smem + isl * STB + wq * 4 * 1024;
        const unsigned kpen = (ilive && ikk < ikn && ik0 + dc * 8 < N) ? 0u : 0x80000000u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, TRIMUL_LDS_PTR(st + i * 1024), 16,
                                                     (oa_t + i * 16u * ROWB + ikb) | kpen, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, TRIMUL_LDS_PTR(st + OPB + i * 1024), 16,
                (ob_t + (32u * (i >> 1) + 4u * (i & 1)) * ROWB + ikb) | kpen, 0, 0, 0);
        }
    };

    const int rchunk = lane >> 4;
    const int fa_base = slot_off(wm * WM + (lane & 15), rchunk);
    const int fb_base = OPB + slot_off(wn * WN + (lane & 15), rchunk);

    f32x4 acc[MB][NB];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 fa[2][MB], fb[2][NB];
    auto barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    // Prologue: group 1 loads steps 0 and 2, group 0 step 1; then the cursor
    // of each group stands on its first step of the loop (3 or 4).
    if (wm == 1) {
        issue(); advance(); advance();
        issue(); advance(); advance();
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(DPW));    // step 0 landed (own share)
    } else {
        advance();
        issue(); advance(); advance();
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));      // step 1 landed (own share)
    }
    barrier();                                          // steps 0 and 1 landed for everyone
    if (wm == 1) barrier();                             // group 1 starts one phase late

    int kin = 0;                                        // super-step within the current tile
    int tl = 0;
    int nk2;                                            // super-steps of tile tl
    {
        size_t bc; int ti, tj, klo, kn; bool lv;
        tile_geo(0, bc, ti, tj);
        krange(bc, ti, tj, klo, kn, lv);
        nk2 = (kn + 1) >> 1;
    }
    int rsl = 0;                                        // ring slot of the current super-step's first step
    for (;;) {
        // M_u: fragments of steps 2u and 2u + 1, then this group's next step.
        const unsigned char* st0 = smem + rsl * STB;
        if (++rsl == NSP) rsl = 0;
        const unsigned char* st1 = smem + rsl * STB;
        if (++rsl == NSP) rsl = 0;
#pragma unroll
        for (int m = 0; m < MB; ++m) fa[0][m] = *reinterpret_cast<const u32x4*>(st0 + fa_base + m * 1024);
#pragma unroll
        for (int n = 0; n < NB; ++n) fb[0][n] = *reinterpret_cast<const u32x4*>(st0 + fb_base + n * 1024);
#pragma unroll
        for (int m = 0; m < MB; ++m) fa[1][m] = *reinterpret_cast<const u32x4*>(st1 + fa_base + m * 1024);
#pragma unroll
        for (int n = 0; n < NB; ++n) fb[1][n] = *reinterpret_cast<const u32x4*>(st1 + fb_base + n * 1024);
        issue();
        advance();
        advance();
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds0(DPW));   // all but the step just issued
        barrier();
        // C_u.  Operands swapped (b rows as the MFMA's A): each lane's four
        // results are four consecutive j of one i.
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int n = 0; n < NB; ++n) acc[m][n] = Elem<bf16>::mma(fb[h][n], fa[h][m], acc[m][n]);
        if (wm == 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));     // its step of the next super-step
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(DPW));
        barrier();
        if (++kin == nk2) {
            // Tile tl complete: store this wave's block and start the next.
            size_t bc; int ti, tj;
            tile_geo(tl, bc, ti, tj);
            const int i0 = ti * TB, j0 = tj * TB;
            bf16* Ob = args.O + bc * args.o_stride;
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                const int i = i0 + wm * WM + m * 16 + (lane & 15);
#pragma unroll
                for (int p = 0; p < NB / 2; ++p) {
                    // j .. j + 7 (8 divides N, so all or none exist)
                    const int j = j0 + wn * WN + 32 * p + 8 * (lane >> 4);
                    bf16x8 h;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        h[e] = (bf16)acc[m][2 * p][e];
                        h[4 + e] = (bf16)acc[m][2 * p + 1][e];
                    }
                    if (i < N && j < N) *reinterpret_cast<bf16x8*>(Ob + (size_t)i * N + j) = h;
                    acc[m][2 * p] = f32x4{0.f, 0.f, 0.f, 0.f};
                    acc[m][2 * p + 1] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
            kin = 0;
            if (++tl == n_my) break;
            size_t nbc; int nti, ntj, klo, kn; bool lv;
            tile_geo(tl, nbc, nti, ntj);
            krange(nbc, nti, ntj, klo, kn, lv);
            nk2 = (kn + 1) >> 1;
        }
    }
    if (wm == 0) barrier();                             // balance group 1's extra barrier
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));          // no DMA may outlive the workgroup
}

// ---------------------------------------------------------------------------
// Live key ranges of the contraction's row tiles, read from the pair mask.
//
// Row r, key k of both operands is scaled by M[r][k] = mask[b][r][k]
// (outgoing) or mask[b][k][r] (incoming), so where M is zero for every row of
// a row tile, every product of that tile with that key is an exact zero.
// ranges[b][t] = (lo, hi) in K-steps of 32 keys: every key outside
// [32 lo, 32 hi) is zero for all rows of tile t; (0, 0) if no key is live.
// A mask value counts as live unless it compares equal to zero (-0 is zero,
// NaN is live, so a NaN still reaches the output).
// One 1024-thread workgroup per (tile, batch element) reads the tile's mask
// rows (outgoing) or columns (incoming) once, in 16-byte chunks, eight loads
// in flight per thread (128 KB per workgroup; with 256 threads the scan took
// 13-16 us at N = 384, where each of the two workgroups waited on six rounds
// of loads).
// ---------------------------------------------------------------------------
template <typename T>
__device__ inline bool mask_live(T v) { return v != (T)0; }

constexpr int K0_THREADS = 1024;

template <typename T>
__global__ __launch_bounds__(K0_THREADS) void k0_mask_ranges(const T* __restrict__ mask, int N, int incoming,
                                                             int* __restrict__ ranges, int* __restrict__ hdr)
{
    constexpr int NT = K0_THREADS;
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 4) hdr[threadIdx.x] = 0;
    constexpr int CE = 16 / (int)sizeof(T);        // elements per 16-byte chunk
    const int t = blockIdx.x, b = blockIdx.y, tiles = gridDim.x;
    const int tid = threadIdx.x;
    const T* m = mask + (size_t)b * N * N;
    const int r0 = t * K2_TILE, rows = min(N, r0 + K2_TILE) - r0;   // multiple of 8
    int kmin = 0x7fffffff, kmax = -1;
    // Each thread keeps U independent 16-byte loads in flight; indices past the
    // end load a valid chunk (the first) and are not counted.
    constexpr int U = 8;
    if (!incoming) {
        // Rows r0 .. r0 + rows - 1 of the mask, keys along the row: chunk
        // idx = r * nch + c of the tile's rows.
        const int nch = N / CE, total = rows * nch;
        const T* tile0 = m + (size_t)r0 * N;
        for (int base = tid; base < total; base += NT * U) {
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int idx = min(base + u * NT, total - 1);
                v[u] = ld16(tile0 + (size_t)(idx / nch) * N + (size_t)(idx % nch) * CE);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int idx = base + u * NT;
                if (idx >= total) break;
                const int key0 = (idx % nch) * CE;
                const T* e = reinterpret_cast<const T*>(&v[u]);
#pragma unroll
                for (int q = 0; q < CE; ++q)
                    if (mask_live(e[q])) {
                        kmin = min(kmin, key0 + q);
                        kmax = max(kmax, key0 + q);
                    }
            }
        }
    } else {
        // Columns r0 .. r0 + rows - 1 of every mask row k: key k is live if any
        // of them is.
        const int cpr = rows / CE;                  // chunks per mask row (1 .. 64)
        const int rpi = NT / cpr;                   // mask rows per pass
        const int c = tid % cpr, k0 = tid / cpr;
        if (k0 < rpi)
            for (int kb = k0; kb < N; kb += rpi * U) {
                u32x4 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int k = min(kb + u * rpi, N - 1);
                    v[u] = ld16(m + (size_t)k * N + r0 + c * CE);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int k = kb + u * rpi;
                    if (k >= N) break;
                    const T* e = reinterpret_cast<const T*>(&v[u]);
                    bool live = false;
#pragma unroll
                    for (int q = 0; q < CE; ++q) live |= mask_live(e[q]);
                    if (live) {
                        kmin = min(kmin, k);
                        kmax = max(kmax, k);
                    }
                }
            }
    }
    // Workgroup min / max.
    for (int off = 32; off > 0; off >>= 1) {
        kmin = min(kmin, __shfl_xor(kmin, off));
        kmax = max(kmax, __shfl_xor(kmax, off));
    }
    __shared__ int smin[NT / 64], smax[NT / 64];
    if ((tid & 63) == 0) { smin[tid >> 6] = kmin; smax[tid >> 6] = kmax; }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < NT / 64; ++w) {
            smin[0] = min(smin[0], smin[w]);
            smax[0] = max(smax[0], smax[w]);
        }
        kmin = smin[0];
        kmax = smax[0];
        int* dst = ranges + ((size_t)b * tiles + t) * 2;
        dst[0] = kmax < 0 ? 0 : kmin / K2_KSTEP;
        dst[1] = kmax < 0 ? 0 : kmax / K2_KSTEP + 1;
    }
}

hipError_t launch_mask_ranges(const Params& p, const void* mask, int B, int N, int incoming, int* table,
                              hipStream_t s)
{
    const int tiles = (N + K2_TILE - 1) / K2_TILE;
    int* hdr = table + 2 * (size_t)B * tiles;
    dim3 grid((unsigned)tiles, (unsigned)B);
    if (p.dtype == DType::BF16)
        hipLaunchKernelGGL(k0_mask_ranges<bf16>, grid, dim3(K0_THREADS), 0, s, (const bf16*)mask, N, incoming, table,
                           hdr);
    else
        hipLaunchKernelGGL(k0_mask_ranges<float>, grid, dim3(K0_THREADS), 0, s, (const float*)mask, N, incoming,
                           table, hdr);
    return hipGetLastError();
}

// Each batch's tile pairs, walked as the contraction walks a channel (groups
// of gm row tiles, column by column), split stably into pairs with at least
// one live K-step and the rest; the header gets the largest live count over
// the batches (its clear is done by the range scan, which runs first).  One
// workgroup per batch element; two passes over the T^2 <= 16384 pairs.
__global__ __launch_bounds__(256) void k0_tile_pairs(int* __restrict__ table, int B, int T, int gm)
{
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int* rg = table + (size_t)b * T * 2;
    int* hdr = table + 2 * (size_t)B * T;
    unsigned* pairs = reinterpret_cast<unsigned*>(hdr + 4) + (size_t)b * T * T;
    const int T2 = T * T;
    auto pair_at = [&](int q, int& ti, int& tj) {
        const int first_i = (q / (gm * T)) * gm;
        const int g = min(gm, T - first_i);
        ti = first_i + (q % (gm * T)) % g;
        tj = (q % (gm * T)) / g;
    };
    auto live_at = [&](int ti, int tj) {
        return max(rg[2 * ti], rg[2 * tj]) < min(rg[2 * ti + 1], rg[2 * tj + 1]);
    };
    __shared__ int wl[4], wd[4];
    int cnt = 0;
    for (int q = tid; q < T2; q += 256) {
        int ti, tj;
        pair_at(q, ti, tj);
        cnt += live_at(ti, tj) ? 1 : 0;
    }
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    if (lane == 0) wl[wave] = cnt;
    __syncthreads();
    const int nlive = wl[0] + wl[1] + wl[2] + wl[3];
    __syncthreads();
    int base_l = 0, base_d = nlive;
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int q0 = 0; q0 < T2; q0 += 256) {
        const int q = q0 + tid;
        int ti = 0, tj = 0;
        bool live = false;
        if (q < T2) {
            pair_at(q, ti, tj);
            live = live_at(ti, tj);
        }
        const unsigned long long bl = __ballot(q < T2 && live), bd = __ballot(q < T2 && !live);
        if (lane == 0) {
            wl[wave] = __popcll(bl);
            wd[wave] = __popcll(bd);
        }
        __syncthreads();
        int ol = 0, od = 0, tl = 0, td = 0;
        for (int w = 0; w < 4; ++w) {
            if (w < wave) { ol += wl[w]; od += wd[w]; }
            tl += wl[w];
            td += wd[w];
        }
        if (q < T2) {
            const unsigned e = (unsigned)ti | ((unsigned)tj << 16);
            if (live) pairs[base_l + ol + __popcll(bl & below)] = e;
            else pairs[base_d + od + __popcll(bd & below)] = e;
        }
        base_l += tl;
        base_d += td;
        __syncthreads();
    }
    if (tid == 0) atomicMax(hdr, nlive);
}

hipError_t launch_tile_pairs(const Plan& plan, int* table, int B, int N, hipStream_t s)
{
    if (plan.k2_tile != K2_TILE) return hipSuccess;   // 128-row tiles walk the plain order
    const int tiles = (N + K2_TILE - 1) / K2_TILE;
    hipLaunchKernelGGL(k0_tile_pairs, dim3((unsigned)B), dim3(256), 0, s, table, B, tiles, plan.k2_gm);
    return hipGetLastError();
}

template <typename T, int BM, int BN>
static hipError_t launch_k2(const void* a, const void* b, int N, const ContractJob& job, hipStream_t s)
{
    const int tiles_i = (N + BM - 1) / BM, tiles_j = (N + BN - 1) / BN;
    dim3 grid((unsigned)((size_t)tiles_i * tiles_j * job.nbc));
    hipLaunchKernelGGL((k2_contract<T, BM, BN>), grid, dim3(256), 0, s,
                       (const T*)a, (const T*)b, (T*)job.o, job.o_stride, job.bc0, N, tiles_j);
    return hipGetLastError();
}

hipError_t launch_contract(const Params& p, const Plan& plan, const void* a_cm, const void* b_cm,
                           int B, int N, const ContractJob& job, hipStream_t s)
{
    // bf16: the persistent kernels with the plan's tile side: 256-row tiles
    // (default) run two K-steps per phase (k2_contract_pp2), 128-row tiles,
    // which waste less on ragged edges at small N, one 64-key step per phase
    // (k2_contract_ppp; its 160 KB would not hold two of their steps and the
    // ring); ragged tiles read zeros or rows whose outputs are never stored.
    if (p.dtype == DType::BF16) {
        const int TB = plan.k2_tile == 128 ? 128 : 256;
        const int tiles = (N + TB - 1) / TB;
        const long long total = (long long)tiles * tiles * job.nbc;   // a multiple of 8: 8 | nbc
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess)
            (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        cus &= ~7;                                                      // G a multiple of 8
        const long long pg = total < cus ? total : cus;
        K2PArgs a;
        a.A = (const bf16*)a_cm;
        a.Bm = (const bf16*)b_cm;
        a.O = (bf16*)job.o;
        a.o_stride = job.o_stride;
        const int T = (N + K2_TILE - 1) / K2_TILE;
        a.ranges = job.table;
        a.hdr = job.table ? job.table + 2 * (size_t)B * T : nullptr;
        a.pairs = job.table ? reinterpret_cast<const unsigned*>(job.table + 2 * (size_t)B * T + 4) : nullptr;
        a.N = N;
        a.C = p.C;
        a.total = (int)total;
        a.bc0 = job.bc0;
        a.order = plan.k2_order;
        a.gm = plan.k2_gm;
        const bool mk = job.table != nullptr;
        if (TB == 128) {
            if (mk) hipLaunchKernelGGL((k2_contract_ppp<4, 128, true>), dim3((unsigned)pg), dim3(512), 0, s, a);
            else hipLaunchKernelGGL((k2_contract_ppp<4, 128, false>), dim3((unsigned)pg), dim3(512), 0, s, a);
        } else {
            if (mk) hipLaunchKernelGGL((k2_contract_pp2<true>), dim3((unsigned)pg), dim3(512), 0, s, a);
            else hipLaunchKernelGGL((k2_contract_pp2<false>), dim3((unsigned)pg), dim3(512), 0, s, a);
        }
        return hipGetLastError();
    }
    return launch_k2<float, 128, 128>(a_cm, b_cm, N, job, s);
}

}  // namespace trimul
