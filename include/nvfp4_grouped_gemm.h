/*
 * nvfp4_grouped_gemm.h - C ABI of the NVFP4 block-scaled grouped GEMM for AMD
 * Instinct MI355X (gfx950).
 *
 * Operation (the contraction stated in the mainloop comment of submission
 * 499344 and built as a block-scaled MMA in my_kernel of submission 506336,
 * kernelindex.com "kernelbot nvfp4 group gemm"): for every group g
 *
 *     C_g[m, n, l] = sum_k (a_g[m, k, l] * sfa_g[m, k/16, l])
 *                        * (b_g[n, k, l] * sfb_g[n, k/16, l])
 *
 * accumulated in fp32 and written as fp16 (round to nearest even, overflow to
 * +-inf).
 *
 * Layouts (the operand and scale layouts built in kernel of submission 385043;
 * tensor shapes from the custom_kernel docstring of submission 499344):
 *   A   uint8 [l][m][k/2]  two FP4 E2M1 codes per byte, K-major; the low
 *                          nibble holds the even K element.
 *   B   uint8 [l][n][k/2]  same.
 *   SFA uint8, tiled: one FP8 E4M3FN scale per row per 16 K-elements. The byte
 *       of row r, 16-block kb, batch li sits at
 *         li*Mt*Kt*512 + (r/128)*Kt*512 + (kb/4)*512
 *           + (r%32)*16 + ((r/32)%4)*4 + kb%4
 *       with Mt = ceil(m/128) and Kt = ceil(k/64); the tensor is padded to
 *       whole 128-row atoms (see nvfp4_sf_bytes). Padded rows are never used.
 *   SFB same with n in place of m.
 *   C   fp16 [l][m][n], row-major.
 *
 * Work decomposition: output tiles (one of a few compiled shapes) are spread
 * over a persistent grid of one workgroup per compute unit, either whole
 * (tiles ordered heaviest first - a group's last tile row, mostly past m,
 * counts as lighter - and dealt out one per workgroup per round, alternately
 * forwards and backwards) or stream-K (each workgroup takes
 * an equal share of all (tile, 128-K stage) units and stores the fp32 partial
 * sums of the tiles it shares; the contributors of a shared tile add their
 * partials pairwise along a fixed binary tree, each node's sum formed by the
 * second of its two children to arrive, so results do not depend on timing,
 * and no workgroup waits for another). Stream-K needs a workspace of two fp32
 * tile-sized slots and 80 bytes of counters per workgroup; a small kernel on
 * the same stream clears the counters first, so the workspace holds no state
 * between calls.
 *
 * Ownership and threading: the caller owns every buffer, the workspace
 * included; the library allocates no device memory and makes no synchronising
 * HIP call, so every entry point can be captured in a HIP graph. Host tables
 * are read before a call returns. Calls are stream-ordered and asynchronous.
 * The library's global state is a per-device cache of the compute-unit count
 * and a per-thread cache of the last eight plans (keyed by the problem sizes,
 * the compute units, the forced choices and the workspace size; no buffer
 * address is kept). Without a workspace (nvfp4_grouped_gemm,
 * nvfp4_grouped_gemm_config, or a NULL workspace) a call uses whole tiles.
 */
#ifndef NVFP4_GROUPED_GEMM_H
#define NVFP4_GROUPED_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_MAX_GROUPS 8

/* Return codes. */
#define NVFP4_OK 0
#define NVFP4_ERR_INVALID (-1)    /* bad group count, size, divisibility or null pointer */
#define NVFP4_ERR_MISALIGNED (-2) /* a device pointer is not 16-byte aligned */
#define NVFP4_ERR_HIP (-3)        /* the HIP runtime reported an error; see nvfp4_last_hip_error */
#define NVFP4_ERR_CONFIG (-4)     /* unknown tile configuration id or split mode */
#define NVFP4_ERR_WORKSPACE (-5)  /* stream-K requested without a large enough workspace (or scratch) */

/*
 * nvfp4_grouped_gemm - run the grouped GEMM on `stream`.
 *
 *   problem_sizes  host int32 [num_groups][4] = (m, n, k, l) per group.
 *   ptrs_abc       host uint64 [num_groups][3] = device addresses of A, B, C.
 *   ptrs_sfa_sfb   host uint64 [num_groups][2] = device addresses of SFA, SFB.
 *   num_groups     1 .. NVFP4_MAX_GROUPS.
 *   stream         a hipStream_t (NULL = the default stream).
 *
 * Requirements, checked before any HIP call (else NVFP4_ERR_INVALID or
 * NVFP4_ERR_MISALIGNED, and nothing is launched):
 *   m, n, k >= 0, l >= 1; k % 32 == 0; n % 8 == 0; k <= 2^22; the bytes of
 *   each of A, B, SFA and SFB (all l batches) below 2^31; m*n*l <= 2^40.
 *   For a group with m > 0 and n > 0, C must be
 *   non-null and 16-byte aligned, and when k > 0 also A, B, SFA and SFB.
 * Semantics at the edges: a group with m == 0 or n == 0 leaves C untouched;
 * k == 0 writes C = 0 (the empty sum).
 * Whole tiles only (no workspace); nothing is allocated.
 * Returns NVFP4_OK once the kernel is enqueued, NVFP4_ERR_HIP if the launch
 * failed.
 */
int nvfp4_grouped_gemm(const int32_t* problem_sizes, const uint64_t* ptrs_abc,
                       const uint64_t* ptrs_sfa_sfb, int num_groups, void* stream);

/*
 * nvfp4_grouped_gemm_ex - as nvfp4_grouped_gemm, with the caller's workspace
 * and explicit choices; allocates nothing.
 *   workspace        device buffer (256-byte aligned) or NULL; its contents
 *                    need no initialisation. Calls that may overlap in time
 *                    need distinct workspaces.
 *   workspace_bytes  its size; see nvfp4_workspace_bytes.
 *   tile_config      -1 (heuristic) or 0 .. nvfp4_num_tile_configs()-1.
 *   split_mode       -1 (heuristic), 0 (whole tiles), 1 (stream-K).
 * With split_mode -1 and no (or too small a) workspace the call uses whole
 * tiles; split_mode 1 without enough workspace returns NVFP4_ERR_WORKSPACE.
 */
int nvfp4_grouped_gemm_ex(const int32_t* problem_sizes, const uint64_t* ptrs_abc,
                          const uint64_t* ptrs_sfa_sfb, int num_groups, void* workspace,
                          size_t workspace_bytes, int tile_config, int split_mode, void* stream);

/*
 * nvfp4_grouped_gemm_scratch - as nvfp4_grouped_gemm_ex, for callers that
 * cannot allocate device memory or pass a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * stream-K partials go to a fixed array of NVFP4_SCRATCH_BYTES that the
 * library's code object holds on each device it runs on (until the process
 * ends). The call allocates nothing.
 *   tile_config, split_mode  as nvfp4_grouped_gemm_ex. With split_mode -1 the
 *                  heuristic considers only stream-K plans whose workspace
 *                  (two fp32 tiles and 80 bytes of counters per workgroup)
 *                  fits NVFP4_SCRATCH_BYTES (32 MiB of partials plus 64 KiB);
 *                  split_mode 1 with a plan that needs more returns
 *                  NVFP4_ERR_WORKSPACE and launches nothing.
 * Every call on a device shares that device's array: calls that may overlap
 * in time on one device (other streams, other threads) race and must not be
 * issued. Nothing in the array needs clearing (a call writes every partial it
 * reads, and clears its counters first). The device's array address is looked up once per device, on the
 * first call with that device current. Returns as nvfp4_grouped_gemm_ex
 * (NVFP4_ERR_HIP if the lookup fails).
 */
#define NVFP4_SCRATCH_BYTES (((size_t)32 << 20) + 65536)
int nvfp4_grouped_gemm_scratch(const int32_t* problem_sizes, const uint64_t* ptrs_abc,
                               const uint64_t* ptrs_sfa_sfb, int num_groups, int tile_config,
                               int split_mode, void* stream);

/*
 * nvfp4_grouped_gemm_stages - as nvfp4_grouped_gemm_ex with the depth of the
 * LDS operand pipeline chosen: `stages` 4 (the depth every other entry point
 * uses) or 3. For verification: the results are bitwise identical to those of
 * nvfp4_grouped_gemm_ex with the same tile_config and split_mode (same
 * plan, same per-tile arithmetic), while each LDS buffer is reloaded one stage
 * sooner after its last reads, so a missing wait or barrier between a buffer's
 * readers and its next loads shows up as a difference. Returns
 * NVFP4_ERR_CONFIG for another `stages`, else as nvfp4_grouped_gemm_ex.
 */
int nvfp4_grouped_gemm_stages(const int32_t* problem_sizes, const uint64_t* ptrs_abc,
                              const uint64_t* ptrs_sfa_sfb, int num_groups, void* workspace,
                              size_t workspace_bytes, int tile_config, int split_mode, int stages,
                              void* stream);

/*
 * nvfp4_grouped_gemm_device - the same grouped GEMM with the group tables in
 * device memory, for up to NVFP4_MAX_DEVICE_GROUPS groups. This is the
 * super-batch of submission 506336 (kernelindex.com "kernelbot nvfp4 group
 * gemm", the super-batch build and its compiled 120-group kernel: the groups
 * of 15 benchmark calls merged into one launch, with the problem sizes and
 * tensor addresses read from device pointer tables and each tile's group
 * found by binary search over the tile prefix). The host reads no table, so
 * a captured HIP graph of this call follows whatever the tables hold when it
 * is replayed.
 *
 *   d_problem_sizes  device int32 [num_groups][4] = (m, n, k, l), 16-byte aligned.
 *   d_ptrs_abc       device uint64 [num_groups][3] = addresses of A, B, C, 16-byte aligned.
 *   d_ptrs_sfa_sfb   device uint64 [num_groups][2] = addresses of SFA, SFB, 16-byte aligned.
 *   num_groups       1 .. NVFP4_MAX_DEVICE_GROUPS.
 *   tile_config      0 .. nvfp4_num_tile_configs()-1, or -1 for 256x256 tiles.
 *   d_status         device int32, 4-byte aligned, or NULL: the kernel stores
 *                    there the number of groups it rejected (0: none).
 *   stream           a hipStream_t (NULL = the default stream).
 *
 * Checked on the host (nothing is launched on failure): num_groups, the table
 * pointers (non-null, aligned), tile_config. Checked by the kernel, per group,
 * with the same rules as nvfp4_grouped_gemm plus at most 2^20 tiles of
 * 128x128 per group: a group that fails is rejected - it gets no tiles, its C
 * is left untouched - and counted in *d_status. Whole tiles only, over one
 * workgroup per compute unit, the full tile rows of all groups first, then
 * the groups' last tile rows by how full they are (the kernel sorts by row
 * count only: groups of different k keep their table order within a class);
 * the library allocates nothing.
 * The tables must stay unchanged until the kernel has finished.
 * Results are those of nvfp4_grouped_gemm with the same tile configuration,
 * bit for bit, except on calls whose groups with work all have k > 3968 (32
 * or more 128-K stages): there the by-value entry points' 256x128, 128x256
 * and 128x128 kernels split K over the waves in every tile (the host knows
 * k), while this kernel splits it only in the
 * 256x128 tiles with at most four row blocks below m (as the by-value
 * kernels do on shorter calls), so the fp32 sums differ in rounding order
 * (both stay within the same bound of the exact result);
 * nvfp4_splits_k_over_waves tells which calls those are.
 * Returns NVFP4_OK once enqueued, NVFP4_ERR_HIP if the launch failed.
 */
#define NVFP4_MAX_DEVICE_GROUPS 512
int nvfp4_grouped_gemm_device(const int32_t* d_problem_sizes, const uint64_t* d_ptrs_abc,
                              const uint64_t* d_ptrs_sfa_sfb, int num_groups, int tile_config,
                              int32_t* d_status, void* stream);

/*
 * nvfp4_grouped_gemm_pow2 - the same grouped GEMM for scale tensors whose
 * used scales are all zero or positive powers of two (the E4M3 codes 0x00,
 * 0x01, 0x02, 0x04 and 0x08, 0x10, ..., 0x78: 0 and 2^-9 .. 2^8). Such a
 * scale is an MX (E8M0) scale, so the block-scaled MMA runs as the FP4 matrix
 * instruction with per-lane E8M0 scales and without dequantising. This is the
 * MMA of my_kernel of submission 506336 (kernelindex.com "kernelbot nvfp4
 * group gemm"), an MX/NV FP4 block-scaled operation whose scale type is a
 * parameter, taken with MX-compatible scales at the NVFP4 16-element block.
 * The results equal those of nvfp4_grouped_gemm to the same tolerance (every
 * product is exact; fp32 accumulation order differs); a zero scale may turn
 * an exact zero sum into -0.
 *
 *   Arguments as nvfp4_grouped_gemm_ex (same checks, same plans, allocates
 *   nothing), plus
 *   d_status  device int32, 4-byte aligned, not NULL. The kernel stores 1
 *             there if a scale of a row below m (column below n) and a
 *             16-block below k is not one of the codes above; it stores
 *             nothing otherwise, so the caller clears it before the call.
 *             With 1 there the C of the call is not valid: repeat it with
 *             nvfp4_grouped_gemm. The check also sees the padding rows of a
 *             scale tensor's last 128-row atom (for SFA those in a 32-row
 *             block that also holds rows below m): padding that is not zero
 *             or a power of two (zero padding is) reports 1 as well, which
 *             only costs the fallback. The 16-blocks past k in a half-used
 *             last atom may hold anything.
 * Calls that share d_status and may overlap in time report together.
 * Returns NVFP4_ERR_INVALID for a NULL d_status, NVFP4_ERR_MISALIGNED for a
 * misaligned one, else as nvfp4_grouped_gemm_ex.
 */
int nvfp4_grouped_gemm_pow2(const int32_t* problem_sizes, const uint64_t* ptrs_abc,
                            const uint64_t* ptrs_sfa_sfb, int num_groups, int32_t* d_status,
                            void* workspace, size_t workspace_bytes, int tile_config, int split_mode,
                            void* stream);

/*
 * nvfp4_device_group_tiles - the per-group check of nvfp4_grouped_gemm_device,
 * on the host (no HIP call): `size` = (m, n, k, l), `ptrs` = addresses of
 * (A, B, C, SFA, SFB). Returns the tiles the kernel gives the group with
 * `tile_config` (-1: the default), or -1 if the kernel rejects the group (or
 * an argument is NULL or tile_config unknown).
 */
int64_t nvfp4_device_group_tiles(const int32_t* size, const uint64_t* ptrs, int tile_config);

/*
 * nvfp4_split_plan - how a stream-K call (split mode 1, configuration `cfg`,
 * -1 = heuristic) on `num_cus` compute units divides the work (host only, no
 * HIP call). Tiles are numbered class by class, heaviest first (a group's
 * last tile row, mostly past m, forms a lighter class), and (tile, 128-K
 * stage) units tile by tile. The first *whole_tiles tiles (whole rounds of
 * one tile per workgroup) are dealt out whole; workgroup w (in XCD-major
 * order) then takes units [unit_ranges[w], unit_ranges[w + 1]) of the rest, a
 * range that may be empty. unit_ranges needs max_ranges >= grid + 1 entries
 * (else only *whole_tiles is written). Returns the grid size, or an error.
 */
int nvfp4_split_plan(const int32_t* problem_sizes, int num_groups, int num_cus, int cfg, int32_t* whole_tiles,
                     int32_t* unit_ranges, int max_ranges);

/*
 * nvfp4_workspace_bytes - workspace that covers every plan the library may
 * choose for these sizes on `num_cus` compute units (host only, no HIP call);
 * 0 for invalid sizes.
 */
size_t nvfp4_workspace_bytes(const int32_t* problem_sizes, int num_groups, int num_cus);

/*
 * nvfp4_grouped_gemm_config - as nvfp4_grouped_gemm, with the tile
 * configuration chosen by the caller (0 .. nvfp4_num_tile_configs()-1) instead
 * of by the built-in heuristic; -1 means "heuristic". For tests and tuning.
 * Returns NVFP4_ERR_CONFIG for an unknown id.
 */
int nvfp4_grouped_gemm_config(const int32_t* problem_sizes, const uint64_t* ptrs_abc,
                              const uint64_t* ptrs_sfa_sfb, int num_groups, void* stream,
                              int tile_config);

/*
 * nvfp4_grouped_gemm_validate - the argument checks of nvfp4_grouped_gemm
 * alone. Makes no HIP call (usable without a GPU). Same return codes.
 */
int nvfp4_grouped_gemm_validate(const int32_t* problem_sizes, const uint64_t* ptrs_abc,
                                const uint64_t* ptrs_sfa_sfb, int num_groups);

/* Number of compiled tile configurations. */
int nvfp4_num_tile_configs(void);

/*
 * nvfp4_tile_config_info - tile shape of configuration `cfg`: output tile
 * bm x bn, K-step bk, threads per workgroup. Any output pointer may be NULL.
 * Returns NVFP4_ERR_CONFIG for an unknown id.
 */
int nvfp4_tile_config_info(int cfg, int* bm, int* bn, int* bk, int* threads);

/*
 * nvfp4_select_tile_config - the configuration the heuristic picks for these
 * problem sizes on a device with `num_cus` compute units (host only, no HIP
 * call). Returns a config id, or NVFP4_ERR_INVALID.
 */
int nvfp4_select_tile_config(const int32_t* problem_sizes, int num_groups, int num_cus);

/*
 * nvfp4_launch_geometry - the plan for configuration `cfg` and split mode
 * `split` (-1 = heuristic for either) on `num_cus` compute units, assuming a
 * workspace is available (host only, no HIP call): total output tiles,
 * persistent grid size, whether stream-K is used and the workspace it needs.
 * Any output pointer may be NULL. Returns the config id used, or an error.
 */
int nvfp4_launch_geometry(const int32_t* problem_sizes, int num_groups, int num_cus, int cfg, int split,
                          int64_t* total_tiles, int* grid, int* split_used, size_t* workspace_bytes);

/*
 * nvfp4_splits_k_over_waves - whether nvfp4_grouped_gemm and its _config,
 * _ex, _scratch and _stages forms run the plan for these sizes (configuration
 * `cfg` and split mode `split`, -1 = heuristic, as in nvfp4_launch_geometry)
 * with the kernels that split K over the four waves of every tile: whole
 * tiles of the 256x128, 128x256 or 128x128 configuration, every group with
 * m, n and k > 0 having at least 32 stages of 128 K (k > 3968). Their fp32
 * sums are then added in another order than in the kernels that split K only
 * in light tiles, or not at all (the results differ in the last bits only,
 * within the same bound of the exact result). Host only, no HIP call.
 * Returns 1 or 0, or NVFP4_ERR_INVALID / NVFP4_ERR_CONFIG.
 */
int nvfp4_splits_k_over_waves(const int32_t* problem_sizes, int num_groups, int num_cus, int cfg, int split);

/* Size in bytes of one tiled scale tensor for `rows` rows and `k` K-elements,
 * l batches: ceil(rows/128)*128 * ceil(k/64)*4 * l. Returns 0 if any is < 0. */
size_t nvfp4_sf_bytes(int rows, int k, int l);

/* The hipError_t of the last failed HIP call made by this library on the
 * calling thread (0 if none). */
int nvfp4_last_hip_error(void);

/* Static text for a return code. */
const char* nvfp4_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_GROUPED_GEMM_H */
