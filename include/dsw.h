/*
 * dsw.h -- C ABI of the MI355X (gfx950) serial Markov draft walk library.
 *
 * The operation (from "Keeping the Draft Walk on Chip: One Launch for DSpark's
 * Markov Head", tie-pilot-qxw.github.io, section "The serial part of a
 * parallel drafter"): for each request b and k = 0 .. gamma-1
 *
 *     u        = W1[prev]                                  (r = 256)
 *     logit_k  = bf16( base[b,k,:] + bf16( W2 . u ) )       over the vocabulary V
 *     tok_k    = argmax(logit_k)              if T[b] == 0 (lowest id on ties)
 *              = inverse-CDF sample of softmax(logit_k / T[b]) with uniforms[b,k]
 *     prev     = tok_k                        (prev starts at anchor[b])
 *
 * The double rounding (the GEMV result rounded to bf16 before the add, then
 * the sum rounded again) is the one of SGLang's default walk described in the
 * same section and in section "B200: the bf16 table fits on chip".  Ties go to
 * the smallest token id (section "The idea: make the walk resident").  The
 * sampler is the inverse CDF of vLLM PR #64442 ("fused Markov sampling",
 * section "Details"), driven by caller-supplied uniforms.  Temperatures are
 * read per request on the device, so greedy, sampled and mixed batches share
 * one launch (section "The idea: make the walk resident").
 *
 * All tensors are row-major and contiguous.  bf16 values are IEEE bfloat16
 * bit patterns (uint16_t).  Unless stated otherwise, pointers passed to
 * dsw_walk are DEVICE pointers on the handle's device, owned by the caller;
 * the library never frees or retains them past the call.
 *
 * Errors: every function returns 0 on success or a negative DSW_ERR_* code.
 * Device-side faults (a cross-workgroup wait that exceeded its bound, a token
 * id out of range) cannot be returned by the asynchronous dsw_walk; they latch
 * into a status word that dsw_status() reads.  After any error the contents of
 * tokens and logits are unspecified.
 */
#ifndef DSW_H
#define DSW_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- codes ------------------------------------------------------------- */
#define DSW_OK 0
#define DSW_ERR_NULL -1          /* a required pointer is NULL                       */
#define DSW_ERR_BATCH -2         /* B < 0 or B > B_max                               */
#define DSW_ERR_GAMMA -3         /* gamma < 0 or gamma > gamma_max                   */
#define DSW_ERR_RANK -4          /* r != 256 (the only rank the kernels support)     */
#define DSW_ERR_DTYPE -5         /* unknown W2 dtype, or scale given/missing wrongly */
#define DSW_ERR_VOCAB -6         /* V < 1 or too large for the device               */
#define DSW_ERR_LAUNCH -7        /* the persistent grid cannot be co-resident       */
#define DSW_ERR_HIP -8           /* a HIP runtime call failed                        */
#define DSW_ERR_DEVICE -9        /* no such device                                   */
#define DSW_ERR_PLAN -10         /* no execution plan fits the request              */
#define DSW_ERR_ARG -11          /* another invalid argument                         */
#define DSW_ERR_SCRATCH -12      /* dsw_walk_static: the walk needs more workspace than
                                    its static scratch array holds                  */
/* latched by the device, reported by dsw_status() */
#define DSW_ERR_DEV_TIMEOUT -20  /* a cross-workgroup wait exceeded its bound        */
#define DSW_ERR_DEV_TOKEN -21    /* an anchor or token id was outside [0, V)        */
#define DSW_ERR_DEV_UNIFORMS -22 /* T > 0 for a request but uniforms was NULL       */

/* W2 storage */
#define DSW_BF16 0               /* W2 bf16 [V][r]                                   */
#define DSW_INT8 1               /* W2 int8 [V][r] + one fp32 scale per row [V]:
                                    bias = bf16(scale[v] * fp32 sum_j q[v][j] u[j])
                                    (the int8 table with one fp32 scale per row of
                                    section "V = 248,320: 62% on chip, the rest
                                    streamed").  One request: the rows are
                                    widened to bf16 on chip when the shard is
                                    loaded (exact); more requests keep the codes
                                    and widen them every step               */

/* shard GEMV engines */
#define DSW_ENGINE_VALU 0        /* v_dot2 per lane, one row per lane                */
#define DSW_ENGINE_MFMA 1        /* 16x16x32 bf16 MFMA tiles, up to 16 requests free */

/* execution paths chosen by the planner */
#define DSW_PATH_RESIDENT 0      /* every row on chip (VGPR + LDS), one launch       */
#define DSW_PATH_PARTIAL 1       /* rows on chip + rows streamed every step          */

/* dsw_create flags */
#define DSW_FLAG_FORCE_STREAM 1u /* keep nothing on chip: stream W2 every step      */
#define DSW_FLAG_COOPERATIVE 2u  /* launch cooperatively.  By default the walk is an
                                    ordinary launch of one workgroup per CU whose
                                    size (LDS above half a CU) admits exactly one
                                    workgroup per CU, so on a device not shared
                                    with other kernels the whole grid is resident
                                    (checked with the occupancy API at create).
                                    A cooperative launch guarantees residency on a
                                    shared device but costs ~20 us per launch on
                                    MI355X.  If the grid is ever not resident, the
                                    bounded waits give up and dsw_status() returns
                                    DSW_ERR_DEV_TIMEOUT; the kernel never hangs.    */
#define DSW_FLAG_VALU_GEMV 4u    /* force the VALU shard GEMV                        */
#define DSW_FLAG_MFMA_GEMV 8u    /* force the MFMA shard GEMV.  Without either flag
                                    bf16 rows take the MFMA engine and one int8
                                    request takes the VALU engine (measured
                                    faster on MI355X).                             */
#define DSW_FLAG_BATCHED 16u     /* use the batched kernel for every batch size.  It
                                    serves B > 16 always: requests in groups of 16
                                    on the MFMA engine, one owner workgroup per
                                    request for the exchange                   */
#define DSW_FLAG_SINGLE_ROUND 32u /* round once: logit = bf16(base + fp32 dot)
                                    instead of the default walk's
                                    bf16(base + bf16(dot)) -- the rounding of the
                                    pages' H100 int8 kernel ("Keeping the Draft
                                    Walk on Chip", section "Correctness", Fig. 7)
                                    and of vLLM PR #64442 ("Details").  Applies
                                    to every walk of the handle.              */
#define DSW_FLAG_GUMBEL 64u      /* sampled requests draw by Gumbel-max instead of
                                    the inverse CDF: the token is the smallest id
                                    maximising logit / T - ln(-ln U), one noise
                                    uniform U per request, step and vocabulary
                                    row -- the pages' small-batch sampler
                                    ("Keeping the Draft Walk on Chip", section
                                    "The idea: make the walk resident").  U of
                                    row v, request b, step k: Philox-4x32-10 of
                                    counter (v / 4, 256 k + b, round counter,
                                    0x47554D42) under the key of dsw_set_seed,
                                    word v mod 4, as (2 (w >> 9) + 1) 2^-24.
                                    The uniforms argument is not used.  Needs a
                                    seed: dsw_walk returns DSW_ERR_ARG until
                                    dsw_set_seed(h, seed, 1).  bf16 rows with
                                    double rounding: the kernels the inverse
                                    CDF would use (the batched one from 2
                                    requests).  int8 rows or
                                    DSW_FLAG_SINGLE_ROUND: the all-to-all
                                    kernels only, so with DSW_FLAG_BATCHED or
                                    B_max > 16 dsw_create returns
                                    DSW_ERR_ARG.                               */
#define DSW_FLAG_GRU 128u        /* the GRU serial head ("Keeping the Draft Walk on
                                    Chip", section "Beyond DSpark: other serial
                                    heads"): walks go through dsw_walk_gru.
                                    One bf16 request (B_max = 1); not with
                                    DSW_FLAG_GUMBEL, DSW_FLAG_BATCHED or
                                    DSW_FLAG_VALU_GEMV (DSW_ERR_ARG) or int8
                                    rows (DSW_ERR_DTYPE).                      */
#define DSW_FLAG_RNN 256u        /* the RNN serial head (same section; DSpark's
                                    RNN head, read as the tanh RNN cell):
                                    walks go through dsw_walk_rnn.  The same
                                    limits as DSW_FLAG_GRU, and not with it. */
#define DSW_FLAG_GATED 512u      /* DSpark's gated serial head (same section):
                                    walks go through dsw_walk_gated.  The same
                                    limits as DSW_FLAG_GRU, and not with it
                                    or DSW_FLAG_RNN.                           */
#define DSW_FLAG_DOMINO 1024u    /* Domino's serial head (same section): walks
                                    go through dsw_walk_domino.  The limits of
                                    DSW_FLAG_GRU, one head flag per handle,
                                    gamma_max <= 16 (DSW_ERR_GAMMA) and a grid
                                    of r workgroups (DSW_ERR_PLAN on a device
                                    with fewer CUs).                           */

/* Device description the planner works from.  dsw_device_info() fills it
 * from the HIP runtime; tests may pass invented devices to dsw_plan_compute. */
typedef struct dsw_devinfo {
    int cu_count;            /* compute units                                   */
    int simds_per_cu;        /* 4 on CDNA                                       */
    int wave_size;           /* 64                                              */
    int vgprs_per_simd_lane; /* unified VGPR+AGPR file per SIMD lane (512)     */
    int lds_bytes_per_cu;    /* local data share per CU                         */
    int max_lds_per_block;   /* largest LDS allocation for one workgroup        */
    int xcd_count;           /* accelerator complex dies                        */
    int clock_khz;           /* peak engine clock                               */
    long long l2_bytes;      /* L2 per XCD                                      */
    long long hbm_bytes;     /* device memory                                   */
    int cooperative;         /* cooperative launch supported                    */
} dsw_devinfo;

/* What the planner decided for one (V, r, gamma, B, dtype). */
typedef struct dsw_plan_info {
    int path;                /* DSW_PATH_*                                      */
    int grid;                /* workgroups: one per CU                          */
    int block;               /* threads per workgroup                           */
    int rows_per_wg;         /* vocabulary rows owned by each workgroup         */
    int reg_slots;           /* 256-row groups per workgroup held in VGPRs      */
    int reg_rows;            /* rows per workgroup held in VGPRs                */
    int lds_rows;            /* rows per workgroup held in LDS                  */
    int stream_rows;         /* rows per workgroup re-read every step           */
    int batch_tile;          /* compiled request capacity of the chosen kernel  */
    int lds_bytes;           /* dynamic LDS per workgroup                       */
    long long onchip_bytes;  /* W2 bytes held on chip over the whole grid      */
    long long stream_bytes;  /* W2 bytes re-read per step over the whole grid  */
    long long workspace_bytes; /* device workspace owned by the handle         */
    int engine;              /* DSW_ENGINE_*                                    */
    int tiles_per_wave;      /* MFMA: 16-row tiles per wave                     */
    int reg_tiles;           /* MFMA: tiles per wave held in VGPR/AGPRs         */
    int lds_tiles;           /* MFMA: tiles per wave held in LDS                */
    int max_tiles;           /* MFMA: compiled tiles-per-wave capacity          */
    int static_lds_bytes;    /* the kernel's static LDS (an upper bound)        */
    int w2_dtype;            /* DSW_BF16 or DSW_INT8 (int8: MFMA engine only)    */
    int ring_slots;          /* batched kernel: LDS ring slots (groups in flight) */
    int rows_pad;            /* batched kernel: shard rows padded to 128          */
    int prefetch_tiles;      /* MFMA, one bf16 request: streamed tiles per wave
                                whose rows for the next step are loaded into LDS
                                while the step's keys are exchanged ("Keeping
                                the Draft Walk on Chip", section "V = 248,320:
                                62% on chip, the rest streamed")                */
} dsw_plan_info;

typedef struct dsw_handle* dsw_handle_t;

/* Fill *out from the HIP runtime for `device`.  Host only; no kernel runs. */
int dsw_device_info(int device, dsw_devinfo* out);

/* Pure host function: the plan for a walk of (V, r, gamma, B, w2_dtype) on
 * the described device.  Rows are split in contiguous shards of
 * ceil(V / grid) rows, one per workgroup, as the pages' resident kernel gives
 * each CTA one slice of vocabulary rows (section "The idea: make the walk
 * resident"); each shard is placed in VGPRs first, then LDS, and whatever is
 * left is streamed every step (section "V = 248,320: 62% on chip, the rest
 * streamed").  flags: DSW_FLAG_FORCE_STREAM and the engine flags.  One
 * request walking up to 3 steps takes the VALU engine, longer walks the MFMA
 * engine; both keep int8 rows widened to bf16 on chip.  DSW_FLAG_VALU_GEMV
 * with int8 W2 and B > 1 returns DSW_ERR_DTYPE.
 * Returns DSW_ERR_* on invalid sizes or when no plan fits. */
int dsw_plan_compute(const dsw_devinfo* dev, int V, int r, int gamma, int B, int w2_dtype,
                     unsigned flags, dsw_plan_info* out);

/* Create a handle for walks on `device` with vocabulary V, rank r (must be
 * 256), at most gamma_max (1 .. 4096) steps and B_max (1 .. 256) requests per
 * call, and W2 stored as w2_dtype.  The handle holds what the pages' resident
 * kernel keeps between replays ("Keeping the Draft Walk on Chip", section "The
 * idea: make the walk resident": every CTA posts into a shared exchange area,
 * and a round parity lets graph replays run without a memset): it allocates
 * and zeroes the device workspace (per-workgroup mailboxes for both step
 * parities, per-kernel-family launch counters that select the step epochs, a
 * round counter and a status word), and, when the handle can run the batched
 * kernel (B_max >= 2 or DSW_FLAG_BATCHED), about B_max * (V + 16384) * 2
 * bytes (B_max rounded up to 16) where that kernel keeps the current step's
 * logits of its sampled requests for the workgroups that draw their tokens; the
 * handle owns both.  It also checks, with the
 * occupancy API, that every kernel the handle can run fits one workgroup per
 * CU (DSW_ERR_LAUNCH otherwise).  The calling thread's current device is left
 * unchanged. */
int dsw_create(dsw_handle_t* h, int device, int V, int r, int gamma_max, int B_max,
               int w2_dtype, unsigned flags);

/* One round of the walk: one persistent launch on `stream` (a hipStream_t;
 * NULL = the null stream).  Asynchronous: it never waits for the device and
 * allocates nothing.  Argument layout (all device pointers):
 *   W1        bf16 [V][r]
 *   W2        bf16 [V][r] (DSW_BF16) or int8 [V][r] (DSW_INT8)
 *   w2_scale  f32 [V] for DSW_INT8, must be NULL for DSW_BF16
 *   base      bf16 [B][gamma][V]   base logits of the drafter's parallel pass
 *   anchor    int32 [B]            last accepted token of each request
 *   T         f32 [B]              temperature; exactly 0 = greedy
 *   uniforms  f32 [B][gamma] in [0,1), one per request and step; may be NULL
 *             when every T is 0
 *   tokens    int32 [B][gamma] out: tokens[b][0] follows the anchor
 *   logits    bf16 [B][gamma][V] out, or NULL: the exact values the tokens
 *             were selected from (section "The idea: make the walk resident":
 *             the same bits are handed to the verifier)
 * Rows of base/logits beyond V and entries beyond [B][gamma] are never
 * touched.  One handle serves one stream at a time: calls on one handle must
 * not overlap on the device.  B == 0 or gamma == 0 returns 0 and launches
 * nothing. */
int dsw_walk(dsw_handle_t h, const void* W1, const void* W2, const float* w2_scale,
             const void* base, const int32_t* anchor, const float* T, const float* uniforms,
             int32_t* tokens, void* logits, int B, int gamma, void* stream);

/* One round of the GRU serial head ("Keeping the Draft Walk on Chip", section
 * "Beyond DSpark: other serial heads": the walk with a recurrent state, each
 * head supplying only its state update; DeLS-Spec's head is a GRU).  Handle
 * created with DSW_FLAG_GRU (dsw_walk or dsw_walk_rnn on it returns
 * DSW_ERR_ARG, and this call on another handle too).  For k < gamma, with prev = anchor, then the
 * previous token, and h = h0, then the previous state:
 *   x  = W1[prev]
 *   r  = sigmoid(Wih[0:r] x + bih[0:r] + Whh[0:r] h + bhh[0:r])
 *   z  = sigmoid(Wih[r:2r] x + bih[r:2r] + Whh[r:2r] h + bhh[r:2r])
 *   n  = tanh(Wih[2r:3r] x + bih[2r:3r] + r * (Whh[2r:3r] h + bhh[2r:3r]))
 *   h  = (1 - z) * n + z * h                 (fp32, the standard GRU cell)
 *   logit = bf16(base_k + bf16(W2 bf16(h))), tok as in dsw_walk.
 * Arguments as dsw_walk (B must be 0 or 1; bf16 W2, w2_scale NULL), plus
 * (device pointers):
 *   Wih, Whh  bf16 [3r][r]   the cell's input and recurrent weights, gate
 *                            blocks in the order (r, z, n)
 *   bih, bhh  f32 [3r]       their biases
 *   h0        f32 [r]        the initial state
 *   states    f32 [gamma][r] out, or NULL: the state after every step (the
 *                            last one continues the next round)
 * The state is spread over the workgroups (each updates r / grid elements
 * with its rows of the cell held in LDS) and gathered by every workgroup once
 * per step through epoch-tagged mailboxes.  Asynchronous; allocates nothing. */
int dsw_walk_gru(dsw_handle_t h, const void* W1, const void* W2, const void* Wih, const void* Whh,
                 const float* bih, const float* bhh, const float* h0, const void* base,
                 const int32_t* anchor, const float* T, const float* uniforms, int32_t* tokens,
                 void* logits, float* states, int B, int gamma, void* stream);

/* One round of the RNN serial head ("Keeping the Draft Walk on Chip", section
 * "Beyond DSpark: other serial heads": DSpark's own RNN head).  Handle created
 * with DSW_FLAG_RNN.  As dsw_walk_gru with the tanh RNN cell
 *   h = tanh(Wih x + bih + Whh h + bhh)      (fp32, x = W1[prev])
 * and Wih, Whh bf16 [r][r], bih, bhh f32 [r]. */
int dsw_walk_rnn(dsw_handle_t h, const void* W1, const void* W2, const void* Wih, const void* Whh,
                 const float* bih, const float* bhh, const float* h0, const void* base,
                 const int32_t* anchor, const float* T, const float* uniforms, int32_t* tokens,
                 void* logits, float* states, int B, int gamma, void* stream);

/* One round of DSpark's gated serial head ("Keeping the Draft Walk on Chip",
 * section "Beyond DSpark: other serial heads": one r x r matrix that fits in
 * int8 beside the shard, so every CTA applies it itself and the state needs no
 * exchange).  The pages give no equation; this entry point takes a convex gate
 * between the state and the new token's row, the gate read from the state:
 *   x  = W1[prev]
 *   g  = sigmoid(gate_scale * (Gq h) + gate_bias)   (per element, fp32)
 *   h  = g * h + (1 - g) * x
 *   logit = bf16(base_k + bf16(W2 bf16(h))), tok as in dsw_walk.
 * Handle created with DSW_FLAG_GATED (dsw_walk, dsw_walk_gru and dsw_walk_rnn
 * on it return DSW_ERR_ARG, and this call on another handle too).  Arguments
 * as dsw_walk_gru, with the cell replaced by (device pointers):
 *   Gq          int8 [r][r]  the gate matrix's codes, row-major, 16-byte
 *                            aligned (else DSW_ERR_ARG)
 *   gate_scale  f32 [r]      the codes' row scales
 *   gate_bias   f32 [r]      the gate biases
 * Every workgroup holds Gq in LDS (widened once to bf16, which is exact: 128
 * KiB) and updates the whole state; the gates of step k + 1 are formed on the
 * matrix cores while step k's keys travel.  With V > 196,608 the matrix
 * leaves no LDS for the shard, whose rows beyond the registers then stream
 * every step.  Asynchronous; allocates nothing. */
int dsw_walk_gated(dsw_handle_t h, const void* W1, const void* W2, const void* Gq, const float* gate_scale,
                   const float* gate_bias, const float* h0, const void* base, const int32_t* anchor,
                   const float* T, const float* uniforms, int32_t* tokens, void* logits, float* states,
                   int B, int gamma, void* stream);

/* One round of Domino's serial head ("Keeping the Draft Walk on Chip",
 * section "Beyond DSpark: other serial heads": a GRU cell that also reads the
 * drafter's hidden states).  Read here as dsw_walk_gru whose input at step k
 * is the concatenation x = [W1[prev]; H[k]] of the previous token's row and
 * the drafter's hidden state at block position k.  Handle created with
 * DSW_FLAG_DOMINO (the other walk calls refuse it with DSW_ERR_ARG, and this
 * call refuses other handles).  Arguments as dsw_walk_gru except (device
 * pointers):
 *   Wih  bf16 [3r][r + d]  input weights, gate blocks (r, z, n), 16-byte aligned
 *   H    bf16 [gamma][d]   the drafter's hidden states, 16-byte aligned
 *   d                      hidden width: 8 <= d <= 4096, d % 8 == 0
 * (DSW_ERR_ARG otherwise).  Each workgroup forms the hidden states' part of
 * its state element's gate pre-activations for all gamma steps when the walk
 * starts; every step then runs the GRU head's step with that part added.
 * Asynchronous; allocates nothing. */
int dsw_walk_domino(dsw_handle_t h, const void* W1, const void* W2, const void* Wih, const void* Whh,
                    const float* bih, const float* bhh, const float* h0, const void* H, int d,
                    const void* base, const int32_t* anchor, const float* T, const float* uniforms,
                    int32_t* tokens, void* logits, float* states, int B, int gamma, void* stream);

/* Wait for the handle's device, then return and clear the status word that
 * the device latches (0 or a DSW_ERR_DEV_* code).  The pages' kernel bounds
 * every cross-CTA wait ("Keeping the Draft Walk on Chip", section "The idea:
 * make the walk resident": CTAs poll the arrival count); here a wait that
 * exceeds its bound latches DSW_ERR_DEV_TIMEOUT and every workgroup exits.
 * While a device error is latched, later walks on the handle return at once
 * without touching their outputs; after a device error this call re-zeroes
 * the workspace (counters included) so that the next walk starts clean. */
int dsw_status(dsw_handle_t h);

/* The plan dsw_walk uses for batch size B on this handle, for a walk of
 * gamma_max steps (one bf16 request walking up to 3 steps takes the VALU
 * engine instead: see dsw_plan_compute with the walk's own gamma): the
 * slice-per-CTA split and its on-chip / streamed rows of "Keeping the Draft
 * Walk on Chip", sections "The idea: make the walk resident" and "V = 248,320:
 * 62% on chip, the rest streamed".  Host only. */
int dsw_query_plan(dsw_handle_t h, int B, dsw_plan_info* out);

/* Device-drawn uniforms.  With enable != 0, later dsw_walk calls that pass
 * uniforms == NULL draw the uniform of request b at step k on the device:
 * the top 24 bits of word 0 of Philox-4x32-10 (Salmon et al., "Parallel
 * Random Numbers: As Easy as 1, 2, 3", SC 2011) with counter
 * (k, b, round counter, 0x44535721) and key (seed low word, seed high word),
 * times 2^-24.  The round counter is the handle's device counter of completed
 * walks (dsw_round_counter), so every launch or graph replay draws fresh
 * uniforms -- the pages' kernel keys its noise by (seed, row, step, round
 * counter): "Keeping the Draft Walk on Chip", section "The idea: make the
 * walk resident".  Walks that pass uniforms use them.  enable = 0 restores
 * the default (T > 0 with uniforms == NULL is DSW_ERR_DEV_UNIFORMS). */
int dsw_set_seed(dsw_handle_t h, unsigned long long seed, int enable);

/* The handle's device round counter: waits for the device, then reads it.
 * It starts at 0 and counts the walks that completed without a device error;
 * walk n (from 0) draws its device uniforms with round counter n. */
int dsw_round_counter(dsw_handle_t h, unsigned* out);

/* Diagnostics: record per-workgroup, per-step phase timestamps of later
 * dsw_walk calls into `trace`, a device buffer of `bytes` bytes owned by the
 * caller (NULL disables).  Layout: uint64 [grid][gamma+1][8]; row k < gamma
 * holds device-wide 100 MHz clock (s_memrealtime) readings at: step start,
 * inputs staged, GEMV done, workgroup argmax known, key posted, all
 * workgroups arrived, tokens known, and (slot 7) the core-clock counter
 * (s_memtime) at the end of the step; row gamma slot 0 is the kernel's start.
 * Only the first 16 steps are recorded (the timestamps are kept on chip and
 * written once, when the walk ends).  Calls whose trace would not fit in
 * `bytes` record nothing. */
int dsw_set_trace(dsw_handle_t h, void* trace, long long bytes);

/* Diagnostics and tests of the exchange ("Keeping the Draft Walk on Chip",
 * section "The idea: make the walk resident": CTAs post, then poll until
 * every CTA has arrived).  spin_limit: polls before a device wait gives up
 * (0 restores the default, about 2^20); a small value makes the waits give
 * up, which latches DSW_ERR_DEV_TIMEOUT while every workgroup still exits.
 * skew (0 or 1, else DSW_ERR_ARG): 1 makes every workgroup sleep a
 * pseudo-random 0..7 units of ~8k clocks, so that the workgroups reach the
 * rendezvous in a scrambled order: before its first post in the one-kernel
 * exchange (a hook in that kernel's step loop slows every step even when
 * off), before each post of each step in the batched kernel.  Later walks
 * on the handle use both. */
int dsw_set_debug(dsw_handle_t h, unsigned spin_limit, unsigned skew);

/* Tuning: later walks on the handle use `grid` workgroups (1 .. the device's
 * CU count; 0 restores one per CU), so that each owns ceil(V / grid) rows:
 * fewer, larger shards mean fewer participants in every rendezvous and more
 * rows per workgroup (the pages measure their exchange at 0.97 us per step
 * even with 8 CTAs: "Keeping the Draft Walk on Chip", section "B200: the
 * bf16 table fits on chip").  Walks whose shards then exceed the compiled
 * shapes return the planner's error (DSW_ERR_VOCAB); the recurrent heads
 * need a grid of r / 4 (Domino's head: r) workgroups (DSW_ERR_PLAN). */
int dsw_set_grid(dsw_handle_t h, int grid);

/* Test hook: waits for the device, then sets the round counter and both
 * kernel families' launch counters to `value` (e.g. just below a 32-bit
 * wrap of the step sequence numbers). */
int dsw_set_round_counter(dsw_handle_t h, unsigned value);

/* The epoch a mailbox word carries at step sequence number seq (gamma_max
 * times the family's launch count plus the step, mod 2^32): (seq mod 2^27)
 * + 1.  Host only. */
unsigned dsw_debug_epoch(unsigned seq);

/* Diagnostics: out[i] = the Gumbel variate -ln(-ln U) the kernels compute for
 * U = (2 i + 1) 2^-24, for every i < 2^23 (every U of DSW_FLAG_GUMBEL's
 * noise).  out: device buffer of 2^23 floats on the current device; runs
 * asynchronously on `stream`. */
int dsw_debug_gumbel_table(float* out, void* stream);

/* Wait for the handle's device, then free the workspace and the handle (the
 * end of the handle's exchange area, see dsw_create).  NULL is accepted. */
int dsw_destroy(dsw_handle_t h);

/* ---- the allocation-free entry point ------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * dsw_walk_static is dsw_walk without a handle: the same plan, kernels and
 * results for the same (V, dtype, flags, B, gamma), with the workspace in a
 * file-scope device array of the library (36 MiB per GPU, held until the
 * process ends: 4 MiB of mailboxes, counters and status, and 32 MiB where the
 * batched kernel keeps the current step's logits of its sampled requests when
 * `logits` is NULL).  It allocates nothing (no hipMalloc, hipFree or
 * allocating library call) and never waits for the device.
 *   device    the GPU the pointers live on; the call launches there
 *   V, w2_dtype, flags   as dsw_create; flags: DSW_FLAG_FORCE_STREAM,
 *             DSW_FLAG_COOPERATIVE, DSW_FLAG_VALU_GEMV, DSW_FLAG_MFMA_GEMV,
 *             DSW_FLAG_BATCHED, DSW_FLAG_SINGLE_ROUND (others: DSW_ERR_ARG;
 *             sampled requests need `uniforms`)
 *   the tensors, B (0 .. 256), gamma (0 .. 256) and stream   as dsw_walk
 * Errors as dsw_walk, and DSW_ERR_SCRATCH when the planner picks the batched
 * kernel (2 or more requests by default), logits is NULL and
 * ceil(B / 16) * 16 * (V + 16384) * 2 bytes exceed 32 MiB (pass logits, or
 * split the batch).  Every call on a GPU
 * shares that GPU's array and leaves its contents for the next (no clearing
 * is needed between calls): calls that overlap on one GPU race, so issue
 * them one at a time per GPU.  The first call on a device (or
 * dsw_static_init) looks up the array's device address and zero-fills its
 * workspace part with a kernel on the call's stream. */
int dsw_walk_static(int device, int V, int w2_dtype, unsigned flags, const void* W1, const void* W2,
                    const float* w2_scale, const void* base, const int32_t* anchor, const float* T,
                    const float* uniforms, int32_t* tokens, void* logits, int B, int gamma, void* stream);

/* Optional set-up of dsw_walk_static on `device` (call it outside any graph
 * capture): the array's device address and its zero fill, waited for.
 * Allocates nothing. */
int dsw_static_init(int device);

/* dsw_status for dsw_walk_static on `device`: waits for the device, returns
 * and clears the latched device status (0 or a DSW_ERR_DEV_* code); after an
 * error it zero-fills the workspace so that the next call starts clean.
 * Until then later calls on the device return at once, as with a handle. */
int dsw_static_status(int device);

/* Static description of a DSW_* code. */
const char* dsw_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* DSW_H */
