// hfqm.hip -- the HFQM calibration package (.calib.hfq): writer and reader.
//
// Layout (hipfire-calib-data dataset card, ".calib.hfq — HFQM calibration
// package"), little-endian:
//   header, 32 bytes: magic "HFQM", version u32 = 1, arch_id u32, n_entries u32,
//                     metadata_offset u64, data_offset u64;
//   metadata:         one self-delimited JSON value at metadata_offset;
//   index:            n_entries u32, then per entry name_len u16, name (bytes),
//                     quant_type u8, n_dims u8, shape[n_dims] u32, group_size u32,
//                     data_size u64;
//   payloads:         concatenated in index order from data_offset.
// The card leaves the index position implicit: it follows the metadata value
// directly, as the listing orders them, and the payloads follow the index
// directly (readers go by data_offset, so padding would not matter to them).
// A tensor's Hessian is an entry of quant_type 130 (Bf16TrilDiagF32: the
// hessian_pack_tril blob) and its imatrix one of f32 values.  Host code only.
#include "gq.h"
#include "gq_internal.h"

#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

namespace {

constexpr int kMaxDims = 4;

struct Entry {
    std::string name;
    uint8_t qt = 0, nd = 0;
    uint32_t shape[kMaxDims] = {0, 0, 0, 0};
    uint32_t group = 0;
    uint64_t size = 0, offset = 0;     // payload bytes and its byte offset in the file
};

struct Package {
    uint32_t arch = 0;
    uint64_t meta_off = 0, data_off = 0;
    std::string meta;
    std::vector<Entry> entries;
};

template <typename T> void put(std::string &b, T v) { b.append(reinterpret_cast<const char *>(&v), sizeof(T)); }

// Length of the JSON value starting at s[0] (after no leading whitespace), or 0
// if s does not start with an object or array that closes within n bytes.
// Strings are skipped with their escapes; brackets are matched by depth.
size_t json_extent(const char *s, size_t n)
{
    if (n == 0 || (s[0] != '{' && s[0] != '[')) return 0;
    int depth = 0;
    bool str = false;
    for (size_t i = 0; i < n; ++i) {
        const char c = s[i];
        if (str) {
            if (c == '\\') ++i;
            else if (c == '"') str = false;
            continue;
        }
        if (c == '"') str = true;
        else if (c == '{' || c == '[') ++depth;
        else if (c == '}' || c == ']') {
            if (--depth == 0) return i + 1;
        }
    }
    return 0;
}

struct File {
    FILE *f = nullptr;
    explicit File(const char *path, const char *mode) : f(std::fopen(path, mode)) {}
    ~File() { if (f) std::fclose(f); }
};

bool read_at(FILE *f, uint64_t off, void *dst, size_t n)
{
    if (fseeko(f, (off_t)off, SEEK_SET) != 0) return false;
    return std::fread(dst, 1, n, f) == n;
}

// Header, metadata and index of the package at path.
int load(const char *path, Package &p)
{
    if (!path) return gq::set_error(GQ_ERR_INVALID_ARG, "null path");
    File F(path, "rb");
    if (!F.f) return gq::set_error(GQ_ERR_IO, "cannot open the package");
    unsigned char h[32];
    if (!read_at(F.f, 0, h, 32)) return gq::set_error(GQ_ERR_IO, "short header");
    uint32_t version, n;
    if (std::memcmp(h, "HFQM", 4) != 0) return gq::set_error(GQ_ERR_IO, "bad magic (not HFQM)");
    std::memcpy(&version, h + 4, 4);
    std::memcpy(&p.arch, h + 8, 4);
    std::memcpy(&n, h + 12, 4);
    std::memcpy(&p.meta_off, h + 16, 8);
    std::memcpy(&p.data_off, h + 24, 8);
    if (version != 1) return gq::set_error(GQ_ERR_IO, "unsupported HFQM version");
    if (fseeko(F.f, 0, SEEK_END) != 0) return gq::set_error(GQ_ERR_IO, "cannot size the package");
    const uint64_t fsize = (uint64_t)ftello(F.f);
    if (p.meta_off < 32 || p.meta_off > p.data_off || p.data_off > fsize)
        return gq::set_error(GQ_ERR_IO, "offsets out of range");
    // metadata and index both lie in [meta_off, data_off)
    std::vector<char> mi((size_t)(p.data_off - p.meta_off));
    if (!mi.empty() && !read_at(F.f, p.meta_off, mi.data(), mi.size())) return gq::set_error(GQ_ERR_IO, "short metadata");
    const size_t ml = json_extent(mi.data(), mi.size());
    if (ml == 0) return gq::set_error(GQ_ERR_IO, "metadata is not a self-delimited JSON object or array");
    p.meta.assign(mi.data(), ml);
    size_t q = ml;
    auto take = [&](void *dst, size_t k) {
        if (q + k > mi.size()) return false;
        std::memcpy(dst, mi.data() + q, k);
        q += k;
        return true;
    };
    uint32_t n2 = 0;
    if (!take(&n2, 4) || n2 != n) return gq::set_error(GQ_ERR_IO, "index entry count differs from the header's");
    p.entries.assign(n, Entry{});
    uint64_t off = p.data_off;
    for (uint32_t i = 0; i < n; ++i) {
        Entry &e = p.entries[i];
        uint16_t nl = 0;
        if (!take(&nl, 2)) return gq::set_error(GQ_ERR_IO, "truncated index");
        e.name.resize(nl);
        if ((nl && !take(&e.name[0], nl)) || !take(&e.qt, 1) || !take(&e.nd, 1))
            return gq::set_error(GQ_ERR_IO, "truncated index");
        if (e.nd > kMaxDims) return gq::set_error(GQ_ERR_IO, "an entry has more than 4 dimensions");
        for (int d = 0; d < e.nd; ++d)
            if (!take(&e.shape[d], 4)) return gq::set_error(GQ_ERR_IO, "truncated index");
        if (!take(&e.group, 4) || !take(&e.size, 8)) return gq::set_error(GQ_ERR_IO, "truncated index");
        e.offset = off;
        off += e.size;
        if (off > fsize || off < e.offset) return gq::set_error(GQ_ERR_IO, "payloads run past the end of the file");
    }
    return GQ_OK;
}

}  // namespace

extern "C" {

int hfqm_write(const char *path, uint32_t arch_id, const char *metadata_json, int64_t n_entries,
               const char *const *names, const uint8_t *quant_types, const uint8_t *n_dims, const uint32_t *shapes,
               const uint32_t *group_sizes, const uint64_t *data_sizes, const void *const *data)
{
    gq::set_error(GQ_OK, "");
    if (!path || !metadata_json) return gq::set_error(GQ_ERR_INVALID_ARG, "null path or metadata");
    if (n_entries < 0 || n_entries > 0xFFFFFFFFll) return gq::set_error(GQ_ERR_INVALID_ARG, "bad entry count");
    if (n_entries > 0 && (!names || !quant_types || !n_dims || !shapes || !group_sizes || !data_sizes || !data))
        return gq::set_error(GQ_ERR_INVALID_ARG, "null entry array");
    const size_t mlen = std::strlen(metadata_json);
    if (mlen == 0 || json_extent(metadata_json, mlen) != mlen)
        return gq::set_error(GQ_ERR_INVALID_ARG, "metadata must be exactly one JSON object or array");
    std::string idx;
    put<uint32_t>(idx, (uint32_t)n_entries);
    for (int64_t i = 0; i < n_entries; ++i) {
        const size_t nl = names[i] ? std::strlen(names[i]) : 0;
        if (!names[i] || nl > 0xFFFF) return gq::set_error(GQ_ERR_INVALID_ARG, "entry name missing or too long");
        if (n_dims[i] > kMaxDims) return gq::set_error(GQ_ERR_INVALID_ARG, "more than 4 dimensions");
        if (data_sizes[i] > 0 && !data[i]) return gq::set_error(GQ_ERR_INVALID_ARG, "null payload");
        put<uint16_t>(idx, (uint16_t)nl);
        idx.append(names[i], nl);
        put<uint8_t>(idx, quant_types[i]);
        put<uint8_t>(idx, n_dims[i]);
        for (int d = 0; d < n_dims[i]; ++d) put<uint32_t>(idx, shapes[kMaxDims * i + d]);
        put<uint32_t>(idx, group_sizes[i]);
        put<uint64_t>(idx, data_sizes[i]);
    }
    std::string head;
    head.append("HFQM", 4);
    put<uint32_t>(head, 1u);
    put<uint32_t>(head, arch_id);
    put<uint32_t>(head, (uint32_t)n_entries);
    put<uint64_t>(head, 32u);
    put<uint64_t>(head, 32u + mlen + idx.size());
    File F(path, "wb");
    if (!F.f) return gq::set_error(GQ_ERR_IO, "cannot create the package");
    bool ok = std::fwrite(head.data(), 1, head.size(), F.f) == head.size() &&
              std::fwrite(metadata_json, 1, mlen, F.f) == mlen && std::fwrite(idx.data(), 1, idx.size(), F.f) == idx.size();
    for (int64_t i = 0; ok && i < n_entries; ++i)
        ok = data_sizes[i] == 0 || std::fwrite(data[i], 1, (size_t)data_sizes[i], F.f) == data_sizes[i];
    ok = ok && std::fflush(F.f) == 0;
    return ok ? GQ_OK : gq::set_error(GQ_ERR_IO, "write failed");
}

int hfqm_read_header(const char *path, uint32_t *arch_id, int64_t *n_entries, uint64_t *data_offset, char *metadata,
                     size_t metadata_cap, size_t *metadata_len)
{
    gq::set_error(GQ_OK, "");
    Package p;
    const int rc = load(path, p);
    if (rc) return rc;
    if (arch_id) *arch_id = p.arch;
    if (n_entries) *n_entries = (int64_t)p.entries.size();
    if (data_offset) *data_offset = p.data_off;
    if (metadata_len) *metadata_len = p.meta.size();
    if (metadata) {
        if (metadata_cap < p.meta.size() + 1) return gq::set_error(GQ_ERR_INVALID_ARG, "metadata buffer too small");
        std::memcpy(metadata, p.meta.data(), p.meta.size());
        metadata[p.meta.size()] = '\0';
    }
    return GQ_OK;
}

int hfqm_read_entry(const char *path, int64_t i, char *name, size_t name_cap, uint8_t *quant_type, uint8_t *n_dims,
                    uint32_t *shape, uint32_t *group_size, uint64_t *data_size, uint64_t *offset)
{
    gq::set_error(GQ_OK, "");
    Package p;
    const int rc = load(path, p);
    if (rc) return rc;
    if (i < 0 || i >= (int64_t)p.entries.size()) return gq::set_error(GQ_ERR_INVALID_ARG, "entry index out of range");
    const Entry &e = p.entries[(size_t)i];
    if (name) {
        if (name_cap < e.name.size() + 1) return gq::set_error(GQ_ERR_INVALID_ARG, "name buffer too small");
        std::memcpy(name, e.name.data(), e.name.size());
        name[e.name.size()] = '\0';
    }
    if (quant_type) *quant_type = e.qt;
    if (n_dims) *n_dims = e.nd;
    if (shape)
        for (int d = 0; d < kMaxDims; ++d) shape[d] = e.shape[d];
    if (group_size) *group_size = e.group;
    if (data_size) *data_size = e.size;
    if (offset) *offset = e.offset;
    return GQ_OK;
}

int hfqm_read_payload(const char *path, int64_t i, void *dst, size_t dst_bytes)
{
    gq::set_error(GQ_OK, "");
    Package p;
    int rc = load(path, p);
    if (rc) return rc;
    if (i < 0 || i >= (int64_t)p.entries.size()) return gq::set_error(GQ_ERR_INVALID_ARG, "entry index out of range");
    const Entry &e = p.entries[(size_t)i];
    if (e.size == 0) return GQ_OK;
    if (!dst || dst_bytes < e.size) return gq::set_error(GQ_ERR_INVALID_ARG, "destination smaller than the payload");
    File F(path, "rb");
    if (!F.f || !read_at(F.f, e.offset, dst, (size_t)e.size)) return gq::set_error(GQ_ERR_IO, "short payload");
    return GQ_OK;
}

}  // extern "C"
