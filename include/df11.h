/*
 * df11.h -- C ABI of the DF11 (DFloat11) codec for one AMD Instinct MI355X (gfx950).
 *
 * The method: "DFloat11: Kompresi inferensi GPU lossless yang mengecilkan LLM
 * menjadi 70% ukurannya" (GeekNews, id.news.hada.io topic 20542).  Section
 * names below are that page's headings.
 *
 * A BF16 weight keeps its sign and 7-bit mantissa verbatim in one
 * PackedSignMantissa byte, while its 8-bit exponent is Huffman-coded into the
 * bit-packed EncodedExponent stream ("Format DFloat11").  Decoding walks a
 * hierarchy of 256-entry LUTs cut from height-8 subtrees of the code tree, the
 * unused exponent values 240..255 acting as pointers to lower LUTs, plus a
 * 256-byte CodeLengths table ("Decoding berbasis LUT hierarkis").  Each GPU
 * thread decodes the codes that start in its own n-byte segment, from a start
 * bit stored in Gaps; each thread block's first output index is stored once
 * ("Kernel GPU 2 tahap dan metadata bantu").
 *
 * Conventions for every function:
 *  - Return value: DF11_OK (0) or a negative df11_status.  Nothing throws across
 *    this ABI.  Validation runs before any write or launch; on failure no output
 *    buffer is written and no work is enqueued.
 *  - The caller owns every buffer, host and device.  The library never
 *    allocates, frees or synchronises device memory, and keeps no global state;
 *    host functions are reentrant.
 *  - Integers in buffers are little-endian; bit streams are MSB-first (bit p of a
 *    stream is bit 7 - p%8 of byte p/8).
 *  - "host" arguments are host pointers, "device" arguments are device pointers
 *    (hipMalloc'd or equivalent) on the current HIP device.
 */
#ifndef DF11_H
#define DF11_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Most elements one stream may hold: 2^32 - 2^16.  The decoders index
 * elements with 32-bit integers; the margin below 2^32 keeps every index
 * they form (a group's rounded chunk end, a wave's run of rounds ahead)
 * below 2^32 as well. */
#define DF11_MAX_ELEMENTS 4294901760ull

typedef enum df11_status {
    DF11_OK = 0,
    DF11_E_INVALID_ARG = -1,        /* null pointer, unsupported layout, bad size argument */
    DF11_E_RESERVED_EXPONENT = -2,  /* input has exponent >= 240 (Inf/NaN or |x| >= 2^113) */
    DF11_E_CODE_TOO_LONG = -3,      /* a Huffman code would exceed 32 bits */
    DF11_E_TOO_MANY_LUTS = -4,      /* the code tree needs more than 16 lower LUTs */
    DF11_E_BUFFER_TOO_SMALL = -5,   /* a caller buffer is smaller than required */
    DF11_E_BAD_STREAM = -6,         /* header fields or codebook are inconsistent */
    DF11_E_TOO_LARGE = -7,          /* N > DF11_MAX_ELEMENTS elements in one stream */
    DF11_E_HIP = -8                 /* a HIP launch or query failed */
} df11_status;

/* Exponent values 240..255 are pointers inside the LUTs, never symbols. */
#define DF11_FIRST_POINTER 240
/* The root LUT plus one lower LUT per pointer value. */
#define DF11_MAX_LUTS 17
/* Longest code; Gaps hold 5-bit offsets in [0, 31]. */
#define DF11_MAX_CODE_LEN 32
/* Size, in uint32 words, of the dynamic-schedule work counters
 * (df11_device_stream.schedule). */
#define DF11_SCHEDULE_WORDS 144
/* Most streams one df11_decompress_batch call decodes. */
#define DF11_MAX_BATCH 16
/* Token rows and smallest row length of df11_linear. */
#define DF11_LINEAR_MAX_TOKENS 8
#define DF11_LINEAR_MIN_IN_FEATURES 512

/* The codebook shared by all tensors of one stream (host, plain data).
 *   code_lengths[e]: Huffman code length of exponent e, 0 if unused
 *                    (the page's CodeLengths table).
 *   codes[e]:        canonical code of e, right-aligned in code_lengths[e] bits.
 *   luts[i][x]:      LUT i indexed by the next 8 bits x.  A value v < 240 is an
 *                    exponent whose code ends within those 8 bits; v >= 240
 *                    points to LUT 256 - v for the following 8 bits.  LUT 0 is
 *                    the root; lower LUTs are numbered by depth, then prefix.
 *   n_luts:          number of LUTs in use (1..17).
 *   max_len:         longest code length (1..32). */
typedef struct df11_codebook {
    uint8_t code_lengths[256];
    uint32_t codes[256];
    uint8_t luts[DF11_MAX_LUTS][256];
    uint32_t n_luts;
    uint32_t max_len;
} df11_codebook;

/* Launch-shape parameters stored in the stream.
 *   bytes_per_thread (n):  EncodedExponent bytes per decoding thread; the
 *                          page's experiments use 8.  The encoder accepts n >= 4;
 *                          the GPU decoder supports n == 8.
 *   threads_per_group (G): threads per output-position block, a multiple of 64;
 *                          the GPU decoder supports G == 256. */
typedef struct df11_layout {
    uint32_t bytes_per_thread;
    uint32_t threads_per_group;
} df11_layout;

/* Stream header (host).  Buffer sizes include zero padding:
 *   enc_bytes     = round_up(n_threads * n, 16) + 16
 *   sm_bytes      = round_up(n_elements, 64)
 *   gaps_bytes    = 4 * (ceil(5 * n_threads / 32) + 1)
 *   out_pos_bytes = 4 * (n_groups + 1)
 * n_threads = ceil(total_bits / (8 n)), n_groups = ceil(n_threads / G).
 * max_group_elems is the largest out_pos[g+1] - out_pos[g]; df11_plan leaves it
 * at its upper bound G * 8n, df11_encode sets the exact value. */
typedef struct df11_header {
    uint64_t n_elements;
    uint64_t total_bits;
    uint32_t bytes_per_thread;
    uint32_t threads_per_group;
    uint64_t n_threads;
    uint64_t n_groups;
    uint32_t n_luts;
    uint32_t max_len;
    uint64_t enc_bytes;
    uint64_t sm_bytes;
    uint64_t gaps_bytes;
    uint64_t out_pos_bytes;
    uint32_t max_group_elems;
    uint32_t reserved;
} df11_header;

/* A stream resident in device memory (the struct itself is host memory).
 *   enc          device, h.enc_bytes     EncodedExponent, zero-padded
 *   sm           device, h.sm_bytes      PackedSignMantissa: sign in bit 7, mantissa in bits 0..6
 *   gaps         device, h.gaps_bytes    5-bit MSB-first start offsets, one per thread
 *   out_pos      device, n_groups + 1    first output index of each group; last entry N
 *   luts         device, n_luts * 256    df11_codebook.luts rows 0..n_luts-1
 *   code_lengths device, 256             df11_codebook.code_lengths
 *   decode_table device, df11_decode_table_bytes(decode_table_bits)
 *                                        built by df11_build_decode_table, or
 *                                        NULL: a caller holding only the page's
 *                                        arrays passes NULL, and every
 *                                        workgroup then derives the same table
 *                                        in LDS from luts and code_lengths
 *                                        (about a microsecond per launch)
 *   decode_table_bits                    index width of decode_table (10..12);
 *                                        0 with a NULL decode_table selects 11
 *   groups_per_workgroup                 launch shape: groups decoded together by one
 *                                        workgroup (1, 2 or 4); 0 picks the default
 *   schedule     device, DF11_SCHEDULE_WORDS uint32, or NULL
 *                                        work counters for dynamic load balancing:
 *                                        zero-filled by the caller once; every
 *                                        launch leaves them zero again.  Launches
 *                                        that share one must not overlap in time
 *                                        (use one per stream of work); within one
 *                                        batched launch, a stream whose counters
 *                                        an earlier stream of the batch also uses
 *                                        runs the static schedule.  NULL
 *                                        selects a static schedule, which is
 *                                        also used for streams too short to
 *                                        gain from balancing.
 *   max_workgroups                       launch at most this many workgroups (0: as
 *                                        many as fit on the GPU at once); a smaller
 *                                        grid leaves CUs to kernels running
 *                                        concurrently on other streams.  A
 *                                        batched launch takes the smallest cap
 *                                        of its streams and still gives every
 *                                        non-empty stream one workgroup, so it
 *                                        launches at most max(cap, streams).
 *   tile_cols                            0: the stream holds its elements in their
 *                                        own order.  Else the stream holds a
 *                                        (N / tile_cols) x tile_cols matrix in
 *                                        MFMA tile order (df11_tile_order;
 *                                        tile_cols a multiple of 32, N a
 *                                        multiple of 64 * tile_cols): the
 *                                        decompress entry points write it back
 *                                        row-major, and df11_matmul takes only
 *                                        such streams. */
typedef struct df11_device_stream {
    df11_header h;
    const uint8_t *enc;
    const uint8_t *sm;
    const uint8_t *gaps;
    const uint32_t *out_pos;
    const uint8_t *luts;
    const uint8_t *code_lengths;
    const void *decode_table;
    uint32_t decode_table_bits;
    uint32_t groups_per_workgroup;
    uint32_t *schedule;
    uint32_t max_workgroups;
    uint32_t tile_cols;
} df11_device_stream;

/* Accumulate the 256-bin exponent histogram of n BF16 words (host).
 * "Format DFloat11": the Huffman tree is built from the exponent distribution;
 * call once per tensor to share one codebook across tensors.
 * bf16: host, n uint16 BF16 bit patterns.  hist: host, 256 counters, accumulated
 * (not cleared).  DF11_E_RESERVED_EXPONENT if any exponent is >= 240
 * ("Decoding berbasis LUT hierarkis": those values are reused as pointers);
 * hist is then left unchanged. */
int df11_histogram(const uint16_t *bf16, uint64_t n, uint64_t hist[256]);

/* Build the codebook from a histogram (host): Huffman code lengths (ties broken
 * by (weight, id) with leaf id = exponent, merged node id = 256 + merge index),
 * canonical codes, CodeLengths and the hierarchical LUTs ("Format DFloat11",
 * "Decoding berbasis LUT hierarkis").  With fewer than two used exponents the
 * smallest unused exponents below 240 are added with weight 0.
 * Errors: DF11_E_RESERVED_EXPONENT (hist[e] > 0 for e >= 240),
 * DF11_E_CODE_TOO_LONG, DF11_E_TOO_MANY_LUTS.  cb is written only on success. */
int df11_build_codebook(const uint64_t hist[256], df11_codebook *cb);

/* Exact buffer sizes for n elements whose exponent histogram is hist (host).
 * Not on the page: the page fixes what the arrays hold, not how a caller
 * sizes them; this lets the caller allocate every buffer of df11_encode
 * before encoding.  hist must be the histogram of exactly the data that
 * df11_encode will see.  Fills every header field; max_group_elems is an
 * upper bound until encode. */
int df11_plan(const df11_codebook *cb, const uint64_t hist[256], uint64_t n, const df11_layout *lay,
              df11_header *h);

/* Encode n BF16 words (host) into caller buffers sized by df11_plan:
 * enc (h->enc_bytes), sm (h->sm_bytes), gaps (h->gaps_bytes), out_pos
 * (h->n_groups + 1 entries).  h must come from df11_plan for this data; on
 * success it is completed (total_bits, max_group_elems).  Every byte of the
 * buffers is written, padding included.
 * "Kernel GPU 2 tahap dan metadata bantu": gap_t is the bit offset of the first
 * code starting at or after bit 8 n t (the end of the stream counts as a code
 * start); out_pos[g] counts the codes that start before thread g G's segment.
 * Errors: DF11_E_RESERVED_EXPONENT, DF11_E_INVALID_ARG (an exponent without a
 * code, or h does not match the data), DF11_E_TOO_LARGE. */
int df11_encode(const df11_codebook *cb, const uint16_t *bf16, uint64_t n, const df11_layout *lay,
                df11_header *h, uint8_t *enc, uint8_t *sm, uint8_t *gaps, uint32_t *out_pos);

/* Reorder a rows x cols row-major BF16 matrix (host) into MFMA tile order,
 * the element order df11_matmul consumes.  Not on the page (the page fixes no
 * element order); the order of this library's matrix-core product.  Position
 * s of the ordered sequence holds W[r][c] with
 *   panel p = s / (64 cols), q = s mod (64 cols)
 *   k-step ks = q / 2048, u = q mod 2048
 *   n-tile nt = u / 512, v = u mod 512, lane l = v / 8, j = v mod 8
 *   r = 64 p + 16 nt + (l mod 16),  c = 32 ks + 8 (l / 16) + j
 * so every 8 consecutive elements are 8 consecutive columns of one row, and
 * each 512-element block is the B operand that the 64 lanes of a gfx950
 * v_mfma_f32_16x16x32_bf16 read for 16 rows x 32 columns of W.
 * w, out: host, rows * cols uint16, not overlapping.  rows a multiple of 64,
 * cols a multiple of 32, else DF11_E_INVALID_ARG. */
int df11_tile_order(const uint16_t *w, uint64_t rows, uint64_t cols, uint16_t *out);

/* Size in bytes of the decode table for index width bits (10..12), 0 if
 * unsupported.  Not on the page: the decode table is this decoder's own
 * derived data (see df11_build_decode_table). */
uint64_t df11_decode_table_bytes(uint32_t bits);

/* Build the GPU decoder's first-level table from the codebook (host).
 * The table is derived data, not part of the compressed format: for every
 * bits-wide window it lists the complete codes at the start of the window
 * (up to five exponents, their start offsets and their total length) so one LDS
 * lookup resolves several short codes; windows whose first code is longer than
 * the index width fall back to the page's LUT hierarchy.  Layout: for each
 * window x, uint32 words 2x (up to four rotated exponents, one per byte) and
 * 2x + 1 (codes << 11 | bits, the fifth exponent in bits 16..23), then one
 * uint16 start mask per window.
 * table: host, df11_decode_table_bytes(bits) bytes. */
int df11_build_decode_table(const df11_codebook *cb, uint32_t bits, void *table, uint64_t table_bytes);

/* Decompress a device-resident stream into out (device, h.n_elements uint16,
 * not aliasing any input), enqueued on hip_stream (a hipStream_t; NULL is the
 * null stream).  Returns after the launch; buffers must stay alive until the
 * stream's work completes.  Every element of out is overwritten with the
 * original BF16 bits ("Kernel GPU 2 tahap dan metadata bantu": per-thread
 * count, block prefix sum, re-decode into an LDS write buffer, coalesced
 * write).  A stream whose header is valid but whose payload is corrupt cannot
 * make the kernel access memory out of bounds; its output is unspecified.
 * Errors: DF11_E_INVALID_ARG (null pointers, unsupported n, G or
 * decode_table_bits), DF11_E_BAD_STREAM (header sizes inconsistent),
 * DF11_E_HIP (launch failed). */
int df11_decompress(const df11_device_stream *s, uint16_t *out, void *hip_stream);

/* Decompress the stream of a whole transformer block -- every linear weight of
 * the block encoded as one stream with a shared codebook -- into one scratch
 * buffer just before the block's forward pass ("Dekompresi per transformer
 * block").  scratch: device, scratch_elems uint16; views into it (element
 * offset, shape) are kept by the caller.  Same kernel and errors as
 * df11_decompress, plus DF11_E_BUFFER_TOO_SMALL if scratch_elems < N. */
int df11_decompress_block(const df11_device_stream *s, uint16_t *scratch, uint64_t scratch_elems,
                          void *hip_stream);

/* Decompress several independent streams -- each with its own codebook,
 * decode table and output -- in one launch, for instance every linear weight
 * of a transformer block encoded with a codebook of its own ("Dekompresi per
 * transformer block" batches a block's matrices into one launch because a
 * single matrix is too small to fill the GPU).  The grid is divided between
 * the streams in proportion to their work.
 *   streams  host array of n_streams device streams (as for df11_decompress);
 *            all non-empty ones must use the same decode_table_bits and
 *            groups_per_workgroup
 *   outs     host array of n_streams device pointers; outs[i] receives
 *            streams[i].h.n_elements uint16, 16-byte aligned, and may not
 *            overlap any other output or any stream's buffers
 * Streams with N = 0 are skipped.  Errors: DF11_E_TOO_LARGE (n_streams >
 * DF11_MAX_BATCH), DF11_E_INVALID_ARG (mismatched table widths or launch
 * shapes, overlapping buffers, or as for df11_decompress), DF11_E_BAD_STREAM,
 * DF11_E_HIP.  Nothing is launched unless every stream is valid. */
int df11_decompress_batch(const df11_device_stream *streams, uint32_t n_streams, uint16_t *const *outs,
                          void *hip_stream);

/* df11_decompress_batch for callers that cannot allocate device memory or
 * own work-counter buffers (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same decode, with each
 * stream's dynamic-schedule counters taken from a fixed device array inside
 * the library (DF11_MAX_BATCH sets of DF11_SCHEDULE_WORDS uint32, 9 KB per
 * GPU, held until the process ends) instead of streams[i].schedule, which is
 * ignored.  The call allocates nothing: it launches a small kernel that zeroes
 * the counters of this call's streams, then the decode, both on hip_stream.
 * Every call on one GPU shares that array, so calls that overlap in time on
 * one GPU race (serialize them, e.g. on one stream).  Arguments, output and
 * errors as for df11_decompress_batch; DF11_E_TOO_LARGE for more than
 * DF11_MAX_BATCH streams, DF11_E_HIP if the array's device address cannot
 * be found. */
int df11_decompress_batch_noalloc(const df11_device_stream *streams, uint32_t n_streams, uint16_t *const *outs,
                                  void *hip_stream);

/* df11_decompress with the decode kernel timed by the GPU: start_event and
 * stop_event (hipEvent_t created by the caller, either may be NULL) are
 * recorded when the kernel itself starts and ends, so hipEventElapsedTime of
 * the pair is the kernel's duration without the launch gap.  Used to measure
 * the decoder; same arguments, output and errors as df11_decompress.  With a
 * stream of N = 0 nothing is launched and the events are not recorded. */
int df11_decompress_timed(const df11_device_stream *s, uint16_t *out, void *hip_stream, void *start_event,
                          void *stop_event);

/* df11_decompress_batch with the batched kernel timed like
 * df11_decompress_timed: start_event and stop_event (either may be NULL) are
 * recorded when the kernel itself starts and ends.  Same arguments, output
 * and errors as df11_decompress_batch; when every stream is empty nothing is
 * launched and the events are not recorded. */
int df11_decompress_batch_timed(const df11_device_stream *streams, uint32_t n_streams, uint16_t *const *outs,
                                void *hip_stream, void *start_event, void *stop_event);

/* y = x W^T with the decompression fused into the matrix product: W is the
 * stream decoded and viewed as an out_features x in_features row-major BF16
 * matrix, and its BF16 values never reach HBM.  The page's section
 * "Dekompresi yang disesuaikan untuk inferensi GPU" decompresses each weight
 * matrix right before its matrix multiplication; the section "Opini Hacker
 * News" suggests a GEMM that decompresses each tile before the arithmetic,
 * which this is for small token counts (token-by-token generation), where the
 * product is bound by reading W.
 *   w             device stream, h.n_elements == out_features * in_features,
 *                 elements in their own (row-major) order: tile_cols == 0
 *   x             device, n_tokens x in_features BF16 (uint16 bit patterns),
 *                 row-major, 16-byte aligned; read only
 *   n_tokens      1 .. DF11_LINEAR_MAX_TOKENS
 *   in_features   a multiple of 8, at least DF11_LINEAR_MIN_IN_FEATURES
 *   y             device, n_tokens x out_features float, row-major, 4-byte
 *                 aligned, overlapping neither x nor the stream's buffers;
 *                 every element is overwritten
 * y[t][r] is the sum over c of x[t][c] * W[r][c], each product exact in float
 * and the sums taken in float in an unspecified order (atomic adds), so the
 * low bits can differ between calls.  Enqueued on hip_stream (a zeroing kernel
 * for y, then the decode kernel); uses w's schedule counters like
 * df11_decompress, so calls sharing a stream descriptor must not overlap in
 * time.  Errors: DF11_E_INVALID_ARG (sizes, alignment, overlap, or as for
 * df11_decompress), DF11_E_BAD_STREAM, DF11_E_TOO_LARGE (n_tokens *
 * out_features >= 2^32), DF11_E_HIP.  With N = 0 (out_features = 0) nothing
 * is launched. */
int df11_linear(const df11_device_stream *w, const uint16_t *x, uint32_t n_tokens, uint32_t in_features,
                uint32_t out_features, float *y, void *hip_stream);

/* df11_linear accumulating into y: y += x W^T, with the same arguments,
 * sums and errors, and no zeroing kernel; y must hold the values to add to
 * (zeros, say, set once for several products that share one buffer). */
int df11_linear_acc(const df11_device_stream *w, const uint16_t *x, uint32_t n_tokens, uint32_t in_features,
                    uint32_t out_features, float *y, void *hip_stream);

/* df11_linear with start_event and stop_event (hipEvent_t, either may be
 * NULL) recorded when the fused kernel itself starts and ends (the zeroing
 * kernel before it is not included), to measure the fused product.  Same
 * arguments, output and errors. */
int df11_linear_timed(const df11_device_stream *w, const uint16_t *x, uint32_t n_tokens, uint32_t in_features,
                      uint32_t out_features, float *y, void *hip_stream, void *start_event, void *stop_event);

/* df11_linear for several weight matrices that multiply the same x -- a
 * transformer block's q, k and v projections, or its gate and up projections
 * -- in one launch, the grid split between them in proportion to their work
 * (small matrices alone cannot fill the GPU).
 *   ws            host array of n_streams device streams (as for df11_linear);
 *                 the non-empty ones must share decode_table_bits
 *   x, n_tokens, in_features   shared by all, as for df11_linear
 *   out_features  host array: rows of each matrix
 *   ys            host array of device outputs, n_tokens x out_features[i]
 *                 floats each, overlapping neither each other, x nor any
 *                 stream's buffers; overwritten
 *   start_event, stop_event   hipEvent_t or NULL, recorded at the fused
 *                 kernel's own start and end
 * One kernel zeroes every output, then one fused kernel runs.  Errors:
 * DF11_E_TOO_LARGE (n_streams > DF11_MAX_BATCH, or the outputs' total
 * >= 2^32 floats), DF11_E_INVALID_ARG (as for df11_linear, mismatched table
 * widths, overlaps), DF11_E_BAD_STREAM, DF11_E_HIP.  Nothing is launched
 * unless every stream is valid. */
int df11_linear_batch(const df11_device_stream *ws, uint32_t n_streams, const uint16_t *x, uint32_t n_tokens,
                      uint32_t in_features, const uint32_t *out_features, float *const *ys, void *hip_stream,
                      void *start_event, void *stop_event);

/* df11_linear_batch accumulating into every output: ys[i] += x W_i^T, with
 * the same arguments and errors and no zeroing kernel. */
int df11_linear_batch_acc(const df11_device_stream *ws, uint32_t n_streams, const uint16_t *x, uint32_t n_tokens,
                          uint32_t in_features, const uint32_t *out_features, float *const *ys, void *hip_stream,
                          void *start_event, void *stop_event);

/* y = x W^T on the matrix cores with the decompression fused in, for any
 * number of tokens: the page's section "Dekompresi yang disesuaikan untuk
 * inferensi GPU" decompresses each weight matrix right before its matrix
 * multiplication and discards the BF16 copy; the section "Opini Hacker News"
 * suggests a GEMM that decompresses each tile before the arithmetic.  Here
 * every decoded 16 x 32 tile of W goes from the decoder's registers straight
 * into v_mfma_f32_16x16x32_bf16 with the matching tile of x; W's BF16 never
 * reaches HBM.
 *   w             device stream in MFMA tile order: tile_cols == in_features
 *                 (df11_tile_order), h.n_elements == out_features * in_features
 *   x             device, n_tokens x in_features BF16, row-major, 16-byte
 *                 aligned, finite values; read only
 *   n_tokens      >= 1; the stream is swept once per 64 tokens (once up to 16,
 *                 32 or 64)
 *   in_features   a multiple of 32;  out_features a multiple of 64
 *   y             device, n_tokens x out_features float, row-major, 4-byte
 *                 aligned, overlapping neither x nor the stream's buffers;
 *                 every element is overwritten
 * y[t][r] is the sum over c of x[t][c] * W[r][c]: products exact in float,
 * sums in float in an unspecified order (partial sums of a row from several
 * workgroups meet in float atomics), so the low bits can differ between
 * calls.  Enqueued on hip_stream: a zeroing kernel for y, then the fused
 * kernel.  Up to 8 tokens, a stream with schedule counters and at least 12
 * super-groups (2 groups) per workgroup sweeps fixed ranges over 95% of them
 * and hands the rest out with its counters (which launches sharing them
 * must not overlap in time, as for df11_decompress); otherwise the counters
 * are not used.  Not on the page (a load-balancing choice).  Errors:
 * DF11_E_INVALID_ARG (sizes, alignment, overlap, a stream not in tile order,
 * or as for df11_decompress), DF11_E_BAD_STREAM, DF11_E_TOO_LARGE
 * (n_tokens * out_features >= 2^32), DF11_E_HIP. */
int df11_matmul(const df11_device_stream *w, const uint16_t *x, uint32_t n_tokens, uint32_t in_features,
                uint32_t out_features, float *y, void *hip_stream);

/* df11_matmul accumulating into y (y += x W^T): no zeroing kernel. */
int df11_matmul_acc(const df11_device_stream *w, const uint16_t *x, uint32_t n_tokens, uint32_t in_features,
                    uint32_t out_features, float *y, void *hip_stream);

/* df11_matmul with start_event and stop_event (hipEvent_t, either may be
 * NULL) recorded when the fused kernel itself starts and ends. */
int df11_matmul_timed(const df11_device_stream *w, const uint16_t *x, uint32_t n_tokens, uint32_t in_features,
                      uint32_t out_features, float *y, void *hip_stream, void *start_event, void *stop_event);

/* df11_matmul for several weight matrices in one launch, each with its own
 * x and y (a transformer block's q, k and v on one x, or gate and up; or
 * every product of a step), the grid split between them in proportion to
 * their work: small matrices alone cannot fill the GPU, and one launch pays
 * one start and one tail.
 *   ws            host array of n_streams device streams, as for df11_matmul;
 *                 the non-empty ones must share decode_table_bits
 *   xs            host array of device x pointers (xs[i]: n_tokens x
 *                 in_features[i] BF16), may repeat
 *   in_features, out_features   host arrays, as for df11_matmul
 *   ys            host array of device outputs, n_tokens x out_features[i]
 *                 floats, overlapping neither each other, any x nor any
 *                 stream's buffers
 *   accumulate    0: every output is overwritten (one zeroing kernel runs
 *                 first); else ys[i] += xs[i] W_i^T
 *   start_event, stop_event   hipEvent_t or NULL, recorded at the fused
 *                 kernel's own start and end
 * The schedule counters serve as for df11_matmul when every non-empty stream
 * qualifies and none shares its counters with an earlier stream of the
 * batch; otherwise the whole launch sweeps fixed ranges.  Errors:
 * DF11_E_TOO_LARGE (n_streams > DF11_MAX_BATCH, the outputs' total >= 2^32
 * floats), as for df11_matmul otherwise.  Nothing is launched unless every
 * stream is valid. */
int df11_matmul_batch(const df11_device_stream *ws, uint32_t n_streams, const uint16_t *const *xs, uint32_t n_tokens,
                      const uint32_t *in_features, const uint32_t *out_features, float *const *ys, int accumulate,
                      void *hip_stream, void *start_event, void *stop_event);

/* ---------------------------------------------------------------------------
 * rANS exponent coder.  The discussion on the page ("Opini Hacker News")
 * names rANS as an entropy coder that suits SIMD-style instruction sets better
 * than Huffman; the page gives no format, so this one is this library's own:
 * the plain static rANS of asymmetric numeral systems (Duda) with 16-bit
 * renormalisation, laid out for 64-lane waves.
 *   - Frequencies f[s] of the exponents sum to M = 2^DF11_RANS_PROB_BITS;
 *     c[s] = f[0] + ... + f[s - 1].  A state x lies in [2^16, 2^32).
 *   - Encoding s: while x >= f[s] * 2^(32 - prob_bits), emit x mod 2^16 and
 *     shift it out; then x = floor(x / f[s]) * M + x mod f[s] + c[s].
 *     Decoding: slot = x mod M, s with c[s] <= slot < c[s] + f[s],
 *     x = f[s] * floor(x / M) + slot - c[s], and if x < 2^16,
 *     x = x * 2^16 + the next word.
 *   - Segments of DF11_RANS_LANES x DF11_RANS_STEPS exponents: lane l of a
 *     segment codes its positions step * lanes + l with a state of its own
 *     (2^16 when encoding starts).  The decoder takes a segment's words step
 *     by step, and within a step in lane order, one per lane whose state fell
 *     below 2^16.  Per segment the stream stores the lanes' start states and
 *     the offset of its words.
 * Sign/mantissa bytes are stored as for DF11 (PackedSignMantissa).
 * ------------------------------------------------------------------------- */
#define DF11_RANS_PROB_BITS 12
#define DF11_RANS_LANES 64
#define DF11_RANS_STEPS 512
/* Entries of the decoder's slot table (M). */
#define DF11_RANS_TABLE_ENTRIES 4096

typedef struct df11_rans_header {
    uint64_t n_elements;  /* N */
    uint64_t n_segments;  /* ceil(N / (lanes * steps)) */
    uint64_t n_words;     /* 16-bit words in the stream */
    uint32_t prob_bits;   /* DF11_RANS_PROB_BITS */
    uint32_t lanes;       /* DF11_RANS_LANES */
    uint32_t steps;       /* DF11_RANS_STEPS */
    uint32_t reserved;
} df11_rans_header;

/* Quantize an exponent histogram to rANS frequencies summing to 2^12 (host):
 * every used exponent gets max(1, floor(hist * M / N)); a sum below M gives
 * the difference to the most frequent exponent (lowest value on ties); while
 * the sum is above M the largest frequency above 1 (lowest value on ties)
 * drops by one.  An empty histogram gives all zeros.  Errors:
 * DF11_E_INVALID_ARG (null pointer), DF11_E_RESERVED_EXPONENT (hist[e] > 0 for
 * e >= 240). */
int df11_rans_quantize(const uint64_t hist[256], uint32_t freq[256]);

/* rANS-encode n BF16 words (host).  freq: from df11_rans_quantize (or any
 * table summing to M that covers every exponent present).  Outputs (host,
 * caller-allocated): states ceil(n / 32768) * 64 uint32; word_offsets
 * ceil(n / 32768) + 1 uint32 (segment g's words are [word_offsets[g],
 * word_offsets[g + 1])); words room for words_cap uint16 (n always suffices);
 * sm n bytes.  h is filled in.  Errors: DF11_E_INVALID_ARG (null pointer, a
 * table not summing to M, an exponent with frequency 0),
 * DF11_E_RESERVED_EXPONENT, DF11_E_BUFFER_TOO_SMALL (words_cap), DF11_E_TOO_LARGE
 * (n > DF11_MAX_ELEMENTS). */
int df11_rans_encode(const uint32_t freq[256], const uint16_t *w, uint64_t n, uint32_t *states,
                     uint32_t *word_offsets, uint16_t *words, uint64_t words_cap, uint8_t *sm, df11_rans_header *h);

/* The decoder's slot table (host): entry k (0 <= k < 4096) is the rotated
 * exponent s of slot k (s >> 1 | (s & 1) << 7) in bits 0-7, f[s] - 1 in bits
 * 8-19 and k - c[s] in bits 20-31.  table: DF11_RANS_TABLE_ENTRIES uint32.
 * Errors: DF11_E_INVALID_ARG (null pointer, a table not summing to M). */
int df11_rans_build_table(const uint32_t freq[256], uint32_t *table);

/* A device-resident rANS stream (buffers are device pointers, owned by the
 * caller).  words holds h.n_words words followed by padding up to a multiple
 * of 8 words plus 8 more (the decoder reads words 8 at a time), 16-byte
 * aligned; sm holds the N sign/mantissa bytes padded to a multiple of 64,
 * 16-byte aligned. */
typedef struct df11_rans_device_stream {
    df11_rans_header h;
    const uint32_t *table;         /* DF11_RANS_TABLE_ENTRIES entries (df11_rans_build_table) */
    const uint32_t *states;        /* h.n_segments * 64 */
    const uint32_t *word_offsets;  /* h.n_segments + 1 */
    const uint16_t *words;
    const uint8_t *sm;
} df11_rans_device_stream;

/* Decode a device-resident rANS stream into out (device, N uint16, 16-byte
 * aligned, not overlapping the stream), enqueued on hip_stream.  Every
 * element of out is overwritten with the original BF16 bits.  A corrupt
 * payload cannot make the kernel access memory out of bounds; its output is
 * unspecified.  Errors: DF11_E_INVALID_ARG (null pointers, alignment, layout
 * fields other than 12 / 64 / 512, overlap), DF11_E_BAD_STREAM (sizes
 * inconsistent), DF11_E_TOO_LARGE, DF11_E_HIP. */
int df11_rans_decompress(const df11_rans_device_stream *s, uint16_t *out, void *hip_stream);

/* df11_rans_decompress with start_event / stop_event (hipEvent_t, either may
 * be NULL) recorded at the decode kernel's own start and end. */
int df11_rans_decompress_timed(const df11_rans_device_stream *s, uint16_t *out, void *hip_stream,
                               void *start_event, void *stop_event);

/* Static, human-readable name of a status code.  Not on the page (the page
 * describes no API); the names are those of enum df11_status. */
const char *df11_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* DF11_H */
