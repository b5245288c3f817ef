// bg_desc_json.cpp -- descriptors as JSON text: bg_desc_from_json and
// bg_desc_to_json (host code only).
//
// A descriptor is a frozen record: identical records owe identical bits
// ("Taming Bitwise Behavior", section 4).  JSON is the form such a record is
// stored in and handed between tools; reading it back must give the same
// record, so the reader is strict: every key must be a known field, every
// value must have the field's type, and any other document is refused with
// BG_E_INVALID.  Unset fields keep the defaults of bg_desc_default_gemm /
// bg_desc_default_reduce.
//
// Document: {"gemm": {...}, "reduce": {...}}, either member optional.
//   gemm:   version, a_type, b_type, acc_type, out_type, partial_type,
//           merge_type ("fp32" | "bf16" | "int8" | "int32"), mfma
//           ("F32_32X32X16_BF16" | "F32_16X16X32_BF16" | "I32_32X32X32_I8" |
//           "I32_16X16X64_I8"), acc_update ("IN_MFMA" | "SEPARATE_ADD"),
//           k_order ("ASCENDING"), short_turn ("LAST" | "FIRST"),
//           k_slot_layout ("CONTIGUOUS" | "STRIDED"), split_k, cut_rule
//           ("UNIT256_REMAINDER_LAST" | "EXPLICIT"), cut_unit, cuts [..],
//           combine ("BALANCED_NEIGHBOURS_FIRST" | "SEQUENTIAL"), odd_rule
//           ("CARRY_LAST"), rounding_point ("AFTER_COMBINE_RNE"), epilogue
//           ("NONE" | "W8A8_POW2"), mfma_profile_hash ("0x" and 16 hex
//           digits), schedule {bm, bn, bk, waves_m, waves_n, load_path,
//           group_m, stages, last_bm, last_bn, last_waves_m, last_waves_n,
//           last_stages}
//   reduce: version, in_type, acc_type, out_type, op ("sum" | "sumsq" |
//           "sum_and_sumsq"), axis ("row" | "col"), leaf_len, leaf_order
//           ("SEQUENTIAL_NO_SEED"), sq_fma ("fused" | "unfused"), tree
//           ("BALANCED"), odd_rule ("CARRY_LAST"), schedule {leaves_per_wg,
//           cols_per_wg}
// Integers are plain JSON integers (no fraction, no exponent).
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <memory>
#include <string>
#include <vector>

#include "../../include/bitgemm.h"

namespace bgjson {

// ---- a small strict JSON reader --------------------------------------------
struct Value {
    enum Kind { NUL, BOOL, INT, STR, ARR, OBJ } kind = NUL;
    bool b = false;
    int64_t i = 0;
    std::string s;
    std::vector<Value> arr;
    std::vector<std::pair<std::string, Value>> obj;  // in document order
};

struct Reader {
    const char* p;
    const char* end;
    std::string err;

    bool fail(const std::string& m)
    {
        if (err.empty()) err = m;
        return false;
    }
    void ws()
    {
        while (p < end && (*p == ' ' || *p == '\t' || *p == '\n' || *p == '\r')) p++;
    }
    bool lit(const char* w)
    {
        const size_t n = strlen(w);
        if ((size_t)(end - p) < n || memcmp(p, w, n) != 0) return false;
        p += n;
        return true;
    }
    bool str(std::string& out)
    {
        if (p >= end || *p != '"') return fail("a string was expected");
        p++;
        while (p < end && *p != '"') {
            const unsigned char c = (unsigned char)*p;
            if (c < 0x20) return fail("control character inside a string");
            if (c == '\\') {
                if (++p >= end) return fail("unterminated escape");
                switch (*p) {
                case '"': out += '"'; break;
                case '\\': out += '\\'; break;
                case '/': out += '/'; break;
                case 'n': out += '\n'; break;
                case 't': out += '\t'; break;
                case 'r': out += '\r'; break;
                case 'b': out += '\b'; break;
                case 'f': out += '\f'; break;
                default: return fail("unsupported escape in a string");
                }
                p++;
            } else {
                out += (char)c;
                p++;
            }
        }
        if (p >= end) return fail("unterminated string");
        p++;
        return true;
    }
    bool num(Value& v)
    {
        const char* q = p;
        bool neg = false;
        if (q < end && *q == '-') neg = true, q++;
        if (q >= end || *q < '0' || *q > '9') return fail("a value was expected");
        if (*q == '0' && q + 1 < end && q[1] >= '0' && q[1] <= '9') return fail("leading zero in a number");
        uint64_t mag = 0;
        while (q < end && *q >= '0' && *q <= '9') {
            const uint64_t d = (uint64_t)(*q - '0');
            if (mag > (UINT64_MAX - d) / 10) return fail("integer out of range");
            mag = mag * 10 + d;
            q++;
        }
        if (q < end && (*q == '.' || *q == 'e' || *q == 'E')) return fail("descriptor numbers are integers");
        if (mag > (uint64_t)INT64_MAX + (neg ? 1u : 0u)) return fail("integer out of range");
        v.kind = Value::INT;
        v.i = neg ? (int64_t)(0 - mag) : (int64_t)mag;
        p = q;
        return true;
    }
    bool value(Value& v, int depth)
    {
        if (depth > 8) return fail("nesting too deep");
        ws();
        if (p >= end) return fail("unexpected end of text");
        if (*p == '{') {
            p++;
            v.kind = Value::OBJ;
            ws();
            if (p < end && *p == '}') {
                p++;
                return true;
            }
            for (;;) {
                ws();
                std::string k;
                if (!str(k)) return false;
                for (const auto& kv : v.obj)
                    if (kv.first == k) return fail("duplicate key \"" + k + "\"");
                ws();
                if (p >= end || *p != ':') return fail("':' expected after a key");
                p++;
                Value c;
                if (!value(c, depth + 1)) return false;
                v.obj.emplace_back(k, std::move(c));
                ws();
                if (p < end && *p == ',') {
                    p++;
                    continue;
                }
                if (p < end && *p == '}') {
                    p++;
                    return true;
                }
                return fail("',' or '}' expected in an object");
            }
        }
        if (*p == '[') {
            p++;
            v.kind = Value::ARR;
            ws();
            if (p < end && *p == ']') {
                p++;
                return true;
            }
            for (;;) {
                Value c;
                if (!value(c, depth + 1)) return false;
                v.arr.push_back(std::move(c));
                ws();
                if (p < end && *p == ',') {
                    p++;
                    continue;
                }
                if (p < end && *p == ']') {
                    p++;
                    return true;
                }
                return fail("',' or ']' expected in an array");
            }
        }
        if (*p == '"') {
            v.kind = Value::STR;
            return str(v.s);
        }
        if (lit("true")) return v.kind = Value::BOOL, v.b = true, true;
        if (lit("false")) return v.kind = Value::BOOL, v.b = false, true;
        if (lit("null")) return v.kind = Value::NUL, true;
        return num(v);
    }
};

// ---- field maps ------------------------------------------------------------
struct Name {
    const char* s;
    uint32_t v;
};
static const Name kDtype[] = {{"fp32", BG_FP32}, {"bf16", BG_BF16}, {"int8", BG_INT8}, {"int32", BG_INT32}};
static const Name kMfma[] = {{"F32_32X32X16_BF16", BG_MFMA_F32_32X32X16_BF16},
                             {"F32_16X16X32_BF16", BG_MFMA_F32_16X16X32_BF16},
                             {"I32_32X32X32_I8", BG_MFMA_I32_32X32X32_I8},
                             {"I32_16X16X64_I8", BG_MFMA_I32_16X16X64_I8}};
static const Name kAccUpdate[] = {{"IN_MFMA", BG_ACC_IN_MFMA}, {"SEPARATE_ADD", BG_ACC_SEPARATE_ADD}};
static const Name kKOrder[] = {{"ASCENDING", BG_K_ASCENDING}};
static const Name kShortTurn[] = {{"LAST", BG_SHORT_TURN_LAST}, {"FIRST", BG_SHORT_TURN_FIRST}};
static const Name kSlots[] = {{"CONTIGUOUS", BG_SLOTS_CONTIGUOUS}, {"STRIDED", BG_SLOTS_STRIDED}};
static const Name kCutRule[] = {{"UNIT256_REMAINDER_LAST", BG_CUT_UNIT_REMAINDER_LAST}, {"EXPLICIT", BG_CUT_EXPLICIT}};
static const Name kCombine[] = {{"BALANCED_NEIGHBOURS_FIRST", BG_COMBINE_BALANCED}, {"SEQUENTIAL", BG_COMBINE_SEQUENTIAL}};
static const Name kOdd[] = {{"CARRY_LAST", BG_ODD_CARRY_LAST}};
static const Name kRounding[] = {{"AFTER_COMBINE_RNE", BG_ROUND_AFTER_COMBINE_RNE}};
static const Name kEpilogue[] = {{"NONE", BG_EPI_NONE}, {"W8A8_POW2", BG_EPI_W8A8_POW2}};
static const Name kOp[] = {{"sum", BG_RED_SUM}, {"sumsq", BG_RED_SUMSQ}, {"sum_and_sumsq", BG_RED_SUM_AND_SUMSQ}};
static const Name kAxis[] = {{"row", BG_AXIS_ROW}, {"col", BG_AXIS_COL}};
static const Name kLeafOrder[] = {{"SEQUENTIAL_NO_SEED", BG_LEAF_SEQUENTIAL_NO_SEED}};
static const Name kSqFma[] = {{"fused", BG_SQ_FUSED}, {"unfused", BG_SQ_UNFUSED}};
static const Name kTree[] = {{"BALANCED", BG_TREE_BALANCED}};

template <size_t N>
static const char* name_of(const Name (&t)[N], uint32_t v)
{
    for (const Name& n : t)
        if (n.v == v) return n.s;
    return nullptr;
}

struct Ctx {
    std::string err;
    bool fail(const std::string& m)
    {
        if (err.empty()) err = m;
        return false;
    }
    template <size_t N>
    bool name(const Value& v, const Name (&t)[N], const std::string& key, uint32_t& out)
    {
        if (v.kind != Value::STR) return fail("\"" + key + "\" must be a string");
        for (const Name& n : t)
            if (v.s == n.s) return out = n.v, true;
        return fail("\"" + key + "\": unknown value \"" + v.s + "\"");
    }
    bool u32(const Value& v, const std::string& key, uint32_t& out)
    {
        if (v.kind != Value::INT || v.i < 0 || v.i > (int64_t)UINT32_MAX)
            return fail("\"" + key + "\" must be an integer in [0, 2^32)");
        out = (uint32_t)v.i;
        return true;
    }
    bool i32(const Value& v, const std::string& key, int32_t& out)
    {
        if (v.kind != Value::INT || v.i < INT32_MIN || v.i > INT32_MAX)
            return fail("\"" + key + "\" must be a 32-bit integer");
        out = (int32_t)v.i;
        return true;
    }
    bool hash(const Value& v, uint64_t& out)
    {
        if (v.kind != Value::STR || v.s.size() != 18 || v.s[0] != '0' || (v.s[1] != 'x' && v.s[1] != 'X'))
            return fail("\"mfma_profile_hash\" must be a string \"0x\" followed by 16 hex digits");
        uint64_t h = 0;
        for (size_t i = 2; i < v.s.size(); i++) {
            const char c = v.s[i];
            int d = c >= '0' && c <= '9' ? c - '0' : c >= 'a' && c <= 'f' ? c - 'a' + 10 : c >= 'A' && c <= 'F' ? c - 'A' + 10 : -1;
            if (d < 0) return fail("\"mfma_profile_hash\" holds a non-hex digit");
            h = (h << 4) | (uint64_t)d;
        }
        out = h;
        return true;
    }
};

static bool gemm_from(Ctx& c, const Value& o, bg_gemm_desc& d)
{
    if (o.kind != Value::OBJ) return c.fail("\"gemm\" must be an object");
    bool have_cuts = false;
    std::vector<int64_t> cuts;
    for (const auto& kv : o.obj) {
        const std::string& k = kv.first;
        const Value& v = kv.second;
        bool ok;
        if (k == "version") ok = c.u32(v, k, d.version);
        else if (k == "a_type") ok = c.name(v, kDtype, k, d.a_type);
        else if (k == "b_type") ok = c.name(v, kDtype, k, d.b_type);
        else if (k == "acc_type") ok = c.name(v, kDtype, k, d.acc_type);
        else if (k == "out_type") ok = c.name(v, kDtype, k, d.out_type);
        else if (k == "partial_type") ok = c.name(v, kDtype, k, d.partial_type);
        else if (k == "merge_type") ok = c.name(v, kDtype, k, d.merge_type);
        else if (k == "mfma") ok = c.name(v, kMfma, k, d.mfma);
        else if (k == "acc_update") ok = c.name(v, kAccUpdate, k, d.acc_update);
        else if (k == "k_order") ok = c.name(v, kKOrder, k, d.k_order);
        else if (k == "short_turn") ok = c.name(v, kShortTurn, k, d.short_turn);
        else if (k == "k_slot_layout") ok = c.name(v, kSlots, k, d.k_slot_layout);
        else if (k == "split_k") ok = c.u32(v, k, d.split_k);
        else if (k == "cut_rule") ok = c.name(v, kCutRule, k, d.cut_rule);
        else if (k == "cut_unit") ok = c.u32(v, k, d.cut_unit);
        else if (k == "combine") ok = c.name(v, kCombine, k, d.combine);
        else if (k == "odd_rule") ok = c.name(v, kOdd, k, d.odd_rule);
        else if (k == "rounding_point") ok = c.name(v, kRounding, k, d.rounding_point);
        else if (k == "epilogue") ok = c.name(v, kEpilogue, k, d.epilogue);
        else if (k == "mfma_profile_hash") ok = c.hash(v, d.mfma_profile_hash);
        else if (k == "cuts") {
            if (v.kind != Value::ARR) return c.fail("\"cuts\" must be an array of integers");
            if (v.arr.size() > BG_MAX_SPLIT + 1) return c.fail("\"cuts\" holds more than 65 points");
            for (const Value& e : v.arr) {
                if (e.kind != Value::INT) return c.fail("\"cuts\" must be an array of integers");
                cuts.push_back(e.i);
            }
            have_cuts = true;
            ok = true;
        } else if (k == "schedule") {
            if (v.kind != Value::OBJ) return c.fail("\"schedule\" must be an object");
            ok = true;
            for (const auto& s : v.obj) {
                const std::string& sk = s.first;
                bg_gemm_schedule& g = d.sched;
                if (sk == "bm") ok = c.i32(s.second, sk, g.bm);
                else if (sk == "bn") ok = c.i32(s.second, sk, g.bn);
                else if (sk == "bk") ok = c.i32(s.second, sk, g.bk);
                else if (sk == "waves_m") ok = c.i32(s.second, sk, g.waves_m);
                else if (sk == "waves_n") ok = c.i32(s.second, sk, g.waves_n);
                else if (sk == "load_path") ok = c.i32(s.second, sk, g.load_path);
                else if (sk == "group_m") ok = c.i32(s.second, sk, g.group_m);
                else if (sk == "stages") ok = c.i32(s.second, sk, g.stages);
                else if (sk == "last_bm") ok = c.i32(s.second, sk, g.last_bm);
                else if (sk == "last_bn") ok = c.i32(s.second, sk, g.last_bn);
                else if (sk == "last_waves_m") ok = c.i32(s.second, sk, g.last_waves_m);
                else if (sk == "last_waves_n") ok = c.i32(s.second, sk, g.last_waves_n);
                else if (sk == "last_stages") ok = c.i32(s.second, sk, g.last_stages);
                else return c.fail("unknown gemm schedule key \"" + sk + "\"");
                if (!ok) return false;
            }
        } else {
            return c.fail("unknown gemm key \"" + k + "\"");
        }
        if (!ok) return false;
    }
    if (have_cuts) {
        // explicit cut points: split_k + 1 of them (checked against split_k
        // here so that a record never holds a cut table of another length)
        if (cuts.size() != (size_t)d.split_k + 1)
            return c.fail("\"cuts\" must hold split_k + 1 points");
        for (size_t i = 0; i < cuts.size(); i++) d.cuts[i] = cuts[i];
    }
    return true;
}

static bool reduce_from(Ctx& c, const Value& o, bg_reduce_desc& d)
{
    if (o.kind != Value::OBJ) return c.fail("\"reduce\" must be an object");
    for (const auto& kv : o.obj) {
        const std::string& k = kv.first;
        const Value& v = kv.second;
        bool ok;
        if (k == "version") ok = c.u32(v, k, d.version);
        else if (k == "in_type") ok = c.name(v, kDtype, k, d.in_type);
        else if (k == "acc_type") ok = c.name(v, kDtype, k, d.acc_type);
        else if (k == "out_type") ok = c.name(v, kDtype, k, d.out_type);
        else if (k == "op") ok = c.name(v, kOp, k, d.op);
        else if (k == "axis") ok = c.name(v, kAxis, k, d.axis);
        else if (k == "leaf_len") ok = c.u32(v, k, d.leaf_len);
        else if (k == "leaf_order") ok = c.name(v, kLeafOrder, k, d.leaf_order);
        else if (k == "sq_fma") ok = c.name(v, kSqFma, k, d.sq_fma);
        else if (k == "tree") ok = c.name(v, kTree, k, d.tree);
        else if (k == "odd_rule") ok = c.name(v, kOdd, k, d.odd_rule);
        else if (k == "schedule") {
            if (v.kind != Value::OBJ) return c.fail("\"schedule\" must be an object");
            ok = true;
            for (const auto& s : v.obj) {
                if (s.first == "leaves_per_wg") ok = c.i32(s.second, s.first, d.sched.leaves_per_wg);
                else if (s.first == "cols_per_wg") ok = c.i32(s.second, s.first, d.sched.cols_per_wg);
                else return c.fail("unknown reduce schedule key \"" + s.first + "\"");
                if (!ok) return false;
            }
        } else {
            return c.fail("unknown reduce key \"" + k + "\"");
        }
        if (!ok) return false;
    }
    return true;
}

// ---- writer ------------------------------------------------------------------
struct Out {
    std::string s;
    bool bad = false;
    template <size_t N>
    void name(const char* key, const Name (&t)[N], uint32_t v)
    {
        const char* n = name_of(t, v);
        if (!n) {
            bad = true;
            return;
        }
        s += std::string("\"") + key + "\": \"" + n + "\", ";
    }
    void num(const char* key, long long v) { s += std::string("\"") + key + "\": " + std::to_string(v) + ", "; }
    void trim()
    {
        if (s.size() >= 2 && s.compare(s.size() - 2, 2, ", ") == 0) s.resize(s.size() - 2);
    }
};

}  // namespace bgjson

namespace bg {
bg_status json_fail(bg_status s, const std::string& msg);  // bg_api.hip: sets bg_last_error()
}

using namespace bgjson;

extern "C" {

bg_status bg_desc_from_json(const char* json, bg_gemm_desc* g, bg_reduce_desc* r)
{
    if (!json) return bg::json_fail(BG_E_INVALID, "JSON text is NULL");
    if (!g && !r) return bg::json_fail(BG_E_INVALID, "no descriptor to fill");
    Reader rd{json, json + strlen(json), {}};
    Value doc;
    if (!rd.value(doc, 0)) return bg::json_fail(BG_E_INVALID, "malformed JSON: " + rd.err);
    rd.ws();
    if (rd.p != rd.end) return bg::json_fail(BG_E_INVALID, "malformed JSON: text after the document");
    if (doc.kind != Value::OBJ) return bg::json_fail(BG_E_INVALID, "the document must be an object");
    bg_gemm_desc gd;
    bg_reduce_desc rdd;
    if (bg_desc_default_gemm(&gd) != BG_OK || bg_desc_default_reduce(&rdd) != BG_OK)
        return bg::json_fail(BG_E_INVALID, "defaults unavailable");
    Ctx c;
    for (const auto& kv : doc.obj) {
        bool ok;
        if (kv.first == "gemm") ok = gemm_from(c, kv.second, gd);
        else if (kv.first == "reduce") ok = reduce_from(c, kv.second, rdd);
        else return bg::json_fail(BG_E_INVALID, "unknown top-level key \"" + kv.first + "\" (gemm, reduce)");
        if (!ok) return bg::json_fail(BG_E_INVALID, c.err);
    }
    if (g) *g = gd;
    if (r) *r = rdd;
    return BG_OK;
}

bg_status bg_desc_to_json(const bg_gemm_desc* g, const bg_reduce_desc* r, char* buf, size_t cap, size_t* len)
{
    if (!g && !r) return bg::json_fail(BG_E_INVALID, "no descriptor to write");
    Out o;
    o.s = "{";
    if (g) {
        o.s += "\"gemm\": {";
        o.num("version", g->version);
        o.name("a_type", kDtype, g->a_type);
        o.name("b_type", kDtype, g->b_type);
        o.name("acc_type", kDtype, g->acc_type);
        o.name("out_type", kDtype, g->out_type);
        o.name("mfma", kMfma, g->mfma);
        o.name("acc_update", kAccUpdate, g->acc_update);
        o.name("k_order", kKOrder, g->k_order);
        o.name("short_turn", kShortTurn, g->short_turn);
        o.name("k_slot_layout", kSlots, g->k_slot_layout);
        o.num("split_k", g->split_k);
        o.name("cut_rule", kCutRule, g->cut_rule);
        o.num("cut_unit", g->cut_unit);
        if (g->cut_rule == BG_CUT_EXPLICIT) {
            if (g->split_k < 1 || g->split_k > BG_MAX_SPLIT) return bg::json_fail(BG_E_INVALID, "split_k out of range");
            o.s += "\"cuts\": [";
            for (uint32_t s = 0; s <= g->split_k; s++)
                o.s += std::to_string((long long)g->cuts[s]) + (s < g->split_k ? ", " : "");
            o.s += "], ";
        }
        o.name("partial_type", kDtype, g->partial_type);
        o.name("merge_type", kDtype, g->merge_type);
        o.name("combine", kCombine, g->combine);
        o.name("odd_rule", kOdd, g->odd_rule);
        o.name("rounding_point", kRounding, g->rounding_point);
        o.name("epilogue", kEpilogue, g->epilogue);
        char h[32];
        snprintf(h, sizeof h, "0x%016llx", (unsigned long long)g->mfma_profile_hash);
        o.s += std::string("\"mfma_profile_hash\": \"") + h + "\", ";
        const bg_gemm_schedule& sc = g->sched;
        o.s += "\"schedule\": {";
        o.num("bm", sc.bm);
        o.num("bn", sc.bn);
        o.num("bk", sc.bk);
        o.num("waves_m", sc.waves_m);
        o.num("waves_n", sc.waves_n);
        o.num("load_path", sc.load_path);
        o.num("group_m", sc.group_m);
        o.num("stages", sc.stages);
        o.num("last_bm", sc.last_bm);
        o.num("last_bn", sc.last_bn);
        o.num("last_waves_m", sc.last_waves_m);
        o.num("last_waves_n", sc.last_waves_n);
        o.num("last_stages", sc.last_stages);
        o.trim();
        o.s += "}}";
        if (r) o.s += ", ";
    }
    if (r) {
        o.s += "\"reduce\": {";
        o.num("version", r->version);
        o.name("in_type", kDtype, r->in_type);
        o.name("acc_type", kDtype, r->acc_type);
        o.name("out_type", kDtype, r->out_type);
        o.name("op", kOp, r->op);
        o.name("axis", kAxis, r->axis);
        o.num("leaf_len", r->leaf_len);
        o.name("leaf_order", kLeafOrder, r->leaf_order);
        o.name("sq_fma", kSqFma, r->sq_fma);
        o.name("tree", kTree, r->tree);
        o.name("odd_rule", kOdd, r->odd_rule);
        o.s += "\"schedule\": {";
        o.num("leaves_per_wg", r->sched.leaves_per_wg);
        o.num("cols_per_wg", r->sched.cols_per_wg);
        o.trim();
        o.s += "}}";
    }
    o.s += "}";
    if (o.bad) return bg::json_fail(BG_E_INVALID, "a field holds a value that has no name");
    if (len) *len = o.s.size();
    if (!buf || cap < o.s.size() + 1) return bg::json_fail(BG_E_INVALID, "buffer too small: *len holds the length");
    memcpy(buf, o.s.c_str(), o.s.size() + 1);
    return BG_OK;
}

}  // extern "C"
